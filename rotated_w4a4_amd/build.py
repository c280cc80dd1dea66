"""Build libquarot.so (HIP, gfx950) in-tree with hipcc.

    python -m rotated_w4a4_amd.build        # or: from rotated_w4a4_amd.build import build

Every source is compiled for gfx950 only, with packed-fp32 instruction
generation disabled, and linked into rotated_w4a4_amd/libquarot.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libquarot.so")
SOURCES = ["abi.hip", "had_quant.hip", "gemm.hip", "kv.hip", "decode.hip", "cross_head.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile all HIP sources and link libquarot.so; returns its path."""
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="quarot_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            # hipcc's host pass does not know the packed-fp32 feature; harmless
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print("\n".join(lines), file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

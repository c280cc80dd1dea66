"""Host logic of bench.py that needs no GPU: the one-GPU guard, the mapping
of profiled kernel names to their traffic entries, the HBM counter summary
(plain-copy calibration, medians, one-off launches left out) and the
algorithmic byte count of a decode call."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name,key", [
    ("void quarot::had_quant_kront<24, false, 512, false>(__half const*, long)", "had_quant"),
    ("void quarot::had_quant_kront<24, true, 512, false>(__half const*, long)", "had_quant"),
    ("void quarot::had_quant_kront<24, false, 512, true>(__half const*, long)", "swiglu_had_quant"),
    ("void quarot::had_quant_kront<24, true, 512, true>(__half const*, long)", "swiglu_had_quant"),
    ("void quarot::had_quant_kron<28, false, false, 1024>(__half const*)", "had_quant"),
    ("void quarot::had_quant_kron<24, true, false, 512>(__half const*)", "had_quant"),
    ("void quarot::had_quant_kron<24, false, true, 512>(__half const*)", "swiglu_had_quant"),
    ("void quarot::had_quant_kron<28, true, true, 1024>(__half const*)", "swiglu_had_quant"),
    ("void quarot::had_quant_lds<true>(quarot::LdsArgs)", "swiglu_had_quant"),
    ("void quarot::had_quant_lds<false>(quarot::LdsArgs)", "had_quant"),
    ("void quarot::had_quant_4096_split<false>(__half const*)", "had_quant"),
    ("void quarot::(anonymous namespace)::kv_had_quant_kernel<128, false, 1>(quarot::KvLaunch)",
     "kv_had_quant"),
    ("void quarot::decode_split_kernel<0>(quarot::DecodeArgs)", "kv_decode"),
    ("void quarot::decode_combine_kernel<true>(quarot::CombineArgs)", "kv_decode"),
    ("void quarot::(anonymous namespace)::w4a4_gemm_big_kernel<quarot::BigCfg<2, 2, 128, 128, 4> >()",
     "w4a4_gemm"),
    ("void quarot::(anonymous namespace)::w4a4_gemm_kernel<quarot::GemmCfg<2, 4, 64, 64, 256> >()",
     "w4a4_gemm"),
    ("void quarot::cross_head_quant_kernel<64, false, false>(quarot::CrossArgs)", "cross_head"),
    ("__amd_rocclr_copyBuffer", None),
    ("void at::native::vectorized_elementwise_kernel<4>()", None),
])
def test_kernel_names_map_to_traffic_keys(name, key):
    assert bench.kernel_key(name) == key


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_summary_scales_by_the_copy_and_takes_medians(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    gemm = "void quarot::(anonymous namespace)::w4a4_gemm_kernel<quarot::GemmCfg<2, 4, 64, 64, 256> >()"
    prep = "void quarot::had_quant_4096_split<false>(__half const*)"
    cal_f, cal_w = tmp_path / "cal_f.csv", tmp_path / "cal_w.csv"
    # the copy of COPY_BYTES reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _counter_csv(cal_f, [(copy, "FETCH_SIZE", bench.COPY_BYTES / 2048.0)])
    _counter_csv(cal_w, [(copy, "WRITE_SIZE", bench.COPY_BYTES / 1024.0)])
    wf, ww = tmp_path / "w_f.csv", tmp_path / "w_w.csv"
    # three GEMM dispatches (median 1100 KiB read, 500 written); one rotate+quant
    # dispatch (a one-off, left out)
    _counter_csv(wf, [(gemm, "FETCH_SIZE", 1200.0), (gemm, "FETCH_SIZE", 1000.0),
                      (gemm, "FETCH_SIZE", 1100.0), (prep, "FETCH_SIZE", 9.0)])
    _counter_csv(ww, [(gemm, "WRITE_SIZE", 500.0), (gemm, "WRITE_SIZE", 500.0),
                      (gemm, "WRITE_SIZE", 500.0), (prep, "WRITE_SIZE", 9.0)])
    args = types.SimpleNamespace(traffic_from=[str(cal_f), str(cal_w), "wl", str(wf), str(ww)])
    t = bench.summarize_counters(args)
    assert t["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    ent = t["kernels"]["wl"]
    assert set(ent) == {"w4a4_gemm"}
    g = ent["w4a4_gemm"]
    assert g["fetch_kib"] == 1100.0 and g["write_kib"] == 500.0
    assert g["fetch_bytes"] == pytest.approx(1100.0 * 1024 * 2.0)
    assert g["write_bytes"] == pytest.approx(500.0 * 1024)
    assert g["source_sha256"] == bench.source_digest("w4a4_gemm")
    json.dumps(t)  # the summary is plain JSON


def test_traffic_lookup_needs_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernels": {"wl": {
        "w4a4_gemm": {"source_sha256": bench.source_digest("w4a4_gemm"),
                      "fetch_bytes": 1000.0, "write_bytes": 24.0},
        "had_quant": {"source_sha256": "0" * 64, "fetch_bytes": 1.0, "write_bytes": 1.0}}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("wl", "w4a4_gemm") == 1024
    assert bench.measured_traffic("wl", "had_quant") is None  # sources changed since
    assert bench.measured_traffic("other", "w4a4_gemm") is None


def test_decode_call_bytes_closed_form():
    # 70B grouped-query decode: B 16, 8 KV heads, 64 query heads, 4096 positions,
    # head dim 128; per position and tensor 64 code bytes + a 2-byte scale
    assert bench.decode_call_bytes(16, 8, 64, 4096, 128, 0) == 69_730_304
    # the zero point adds 2 bytes per position and tensor
    assert (bench.decode_call_bytes(16, 8, 64, 4096, 128, 1)
            - bench.decode_call_bytes(16, 8, 64, 4096, 128, 0)) == 2 * 16 * 8 * 4096 * 2

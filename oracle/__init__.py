"""CPU oracle for the rotated W4A4 hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation (float64 / int64) of
what the HIP library computes: randomized Hadamard rotation (Sylvester
H_{2^n}, Kronecker with a Paley H_m), per-token symmetric INT4 quantisation
with nibble packing, the integer GEMM with the per-token x per-channel
dequantisation, the per-head rotation + INT4 quantisation of K/V
(symmetric, and the asymmetric zero-point variant), rotate+quant of the
gated FFN product SiLU(gate) * up, the cross-head transform + quantisation of the attention
output (the out-projection's input), and the decode attention over the INT4 cache with the
cross-head transform (``oracle.attention``).

Only the test suite (``tests/``), the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``rotated_w4a4_amd``) never imports it, and this package imports
nothing from the product path: the two share no code, tables or constants.
Inputs for both come from the seeded generators in ``workloads``.

Every function cites the page passage it follows in its module docstring.
Parity status of each piece (what pins it independently of this code) is
recorded in the test suite; the choice of H_m among all Hadamard matrices of
order m and the random streams are fixed by construction, not by the pages
(parity unpinned for that choice, see ``oracle.hadamard``); every rotation
also takes the caller's H_m as data.
"""

from .hadamard import GF, SUPPORTED_M, hadamard_m, paley1, sylvester
from .rotate import dense_rotation, rotate_rows, split_d
from .quant import (ABSMAX_FLOOR, QMAX, QMIN, ZMAX, asym_codes, asym_params, codes_from_scales,
                    pack_int4, pack_uint4, quantize_rows, quantize_rows_asym, row_scales,
                    unpack_int4, unpack_uint4)
from .gemm import dequant, int_gemm, int_gemm_exact, w4a4_reference
from .pipeline import (cross_head_quant, had_quant, kv_had_quant, kv_had_quant_asym,
                       prep_weights, silu, swiglu, swiglu_had_quant, w4a4_linear)

__all__ = [
    "GF", "SUPPORTED_M", "hadamard_m", "paley1", "sylvester",
    "dense_rotation", "rotate_rows", "split_d",
    "ABSMAX_FLOOR", "QMAX", "QMIN", "codes_from_scales", "pack_int4",
    "quantize_rows", "row_scales", "unpack_int4",
    "ZMAX", "asym_codes", "asym_params", "quantize_rows_asym", "pack_uint4", "unpack_uint4",
    "dequant", "int_gemm", "int_gemm_exact", "w4a4_reference",
    "had_quant", "kv_had_quant", "kv_had_quant_asym", "prep_weights", "w4a4_linear",
    "silu", "swiglu", "swiglu_had_quant", "cross_head_quant",
]

"""Native MXFP4 comparison GEMM (oracle side).

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

MXFP4 is the microscaling format native FP4 hardware takes ("format-aware
fusion" article in the UFP4 page's similar-articles list: the MXFP4 route;
UE5M3 paper, abstract: UE5M3 has to be emulated where the hardware offers
only such power-of-two scales).  Its definition is the OCP Microscaling
specification: E2M1 elements with one E8M0 scale per 32 consecutive
elements along the contraction axis; an E8M0 byte c is 2^(c - 127), and
c = 0xFF is NaN.  Reading: like the UE5M3 GEMM, the comparison GEMM applies
per-tensor scales tsA * tsB to the accumulated sum, so the two differ only
in the block format.

The plain definition: dequantize exactly (q * 2^(c-127) is exact in fp64)
and multiply in fp64.
"""

import numpy as np

from . import formats
from .quantize import unpack_codes

E8M0_BIAS = 127
E8M0_NAN = 0xFF
MX_BLOCK = 32


def e8m0_decode(code):
    """Value of E8M0 code(s) 0..255 as float64 (0xFF -> NaN)."""
    code = np.asarray(code, dtype=np.int64)
    val = np.ldexp(1.0, code - E8M0_BIAS)
    return np.where(code == E8M0_NAN, np.nan, val)


def dequantize_mx(packed, scales):
    """Exact q * 2^(c-127) as float64, shape (n, C); (n, C/2) packed codes
    (element 2j in the low nibble), (n, C/32) E8M0 scales."""
    q = formats.e2m1_decode(unpack_codes(packed))
    s = e8m0_decode(np.asarray(scales, dtype=np.uint8))
    n, c = q.shape
    return (q.reshape(n, c // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(n, c)


def gemm_nt_mx(a_codes, a_scales, ts_a, b_codes, b_scales, ts_b):
    """C = tsA*tsB * A B^T in fp64 on MXFP4 operands, and the per-element
    bound |tsA*tsB| * |A| |B|^T (the GPU tolerance is relative to it)."""
    A = dequantize_mx(a_codes, a_scales)
    B = dequantize_mx(b_codes, b_scales)
    scale = float(np.float32(ts_a)) * float(np.float32(ts_b))
    with np.errstate(invalid="ignore", over="ignore"):
        C = scale * (A @ B.T)
        bound = abs(scale) * (np.abs(A) @ np.abs(B).T)
    return C, bound

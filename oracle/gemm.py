"""The three block-scaled training GEMMs of a linear layer (oracle side).

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

[UFP4] abstract names the three training GEMMs of a linear layer; [UE5M3]
abstract runs them with E2M1/UE5M3 block-16 operands.  For Y = X W^T with
X (tokens x in) and W (out x in):
  fprop  Y  = X  W^T   contraction over in:     A = X  row-wise,   B = W  row-wise
  dgrad  dX = dY W     contraction over out:    A = dY row-wise,   B = W^T (W quantized along out)
  wgrad  dW = dY^T X   contraction over tokens: A = dY^T,          B = X^T (both along tokens)
Every one is C = tsA * tsB * A_q B_q^T with both operands blocked along the
contraction axis ([TIBQ] summary: each operand is quantized along its own
contraction axis).

This is the plain definition, not an algorithm: dequantize both operands
exactly (q * s_b is exact in fp64) and multiply in fp64.  The fp64 product
carries at most K * 2^-53 * sum|a||b| of rounding error, far inside the
1e-5 * sum|a||b| tolerance the GPU result is held to, so the oracle is exact
for that purpose.  Reading: the result is stored as fp32 with both tensor
scales applied to the accumulated sum.
"""

import numpy as np

from .quantize import dequantize_unscaled


def gemm_nt(a_codes, a_scales, ts_a, b_codes, b_scales, ts_b):
    """C = tsA*tsB * A B^T in fp64, and the per-element bound |tsA*tsB| * |A| |B|^T.

    a_codes (M, K/2), a_scales (M, K/16); b_codes (N, K/2), b_scales (N, K/16).
    """
    A = dequantize_unscaled(a_codes, a_scales)
    B = dequantize_unscaled(b_codes, b_scales)
    scale = float(np.float32(ts_a)) * float(np.float32(ts_b))
    C = scale * (A @ B.T)
    bound = abs(scale) * (np.abs(A) @ np.abs(B).T)
    return C, bound


def gemm_nt_entries(a_codes, a_scales, ts_a, b_codes, b_scales, ts_b, rows, cols):
    """The same as gemm_nt but only for entries (rows[t], cols[t]).

    Dequantizes only the rows of A and B involved, so it stays cheap at any
    size.  Returns (values, bounds), each of shape (len(rows),).
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    A = dequantize_unscaled(np.asarray(a_codes)[ur], np.asarray(a_scales)[ur])
    B = dequantize_unscaled(np.asarray(b_codes)[uc], np.asarray(b_scales)[uc])
    scale = float(np.float32(ts_a)) * float(np.float32(ts_b))
    vals = scale * np.einsum("tk,tk->t", A[ri], B[ci])
    bounds = abs(scale) * np.einsum("tk,tk->t", np.abs(A[ri]), np.abs(B[ci]))
    return vals, bounds

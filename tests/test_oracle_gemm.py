"""Pins of the oracle's block-scaled GEMM (the plain definition).

[UFP4] abstract: the three training GEMMs of a linear layer; [UE5M3] abstract:
operands are E2M1 payloads with UE5M3 block-16 scales under tensor scales.
The oracle result is pinned to an exact rational triple loop, to an exact
integer special case, and to what the three GEMMs of a linear layer mean.
"""

from fractions import Fraction

import numpy as np

from oracle import formats, gemm, quantize
from workloads import random_bf16


def _rand_operand(rng, rows, k, scale_lo=0x60, scale_hi=0x90):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(rows, k // 16), dtype=np.uint8)
    return codes, scales


def _exact_value(codes, scales, i, k):
    byte = int(codes[i, k // 2])
    nib = byte & 0xF if k % 2 == 0 else byte >> 4
    q = Fraction(formats.e2m1_decode(nib).item())
    s = Fraction(formats.ue5m3_decode(int(scales[i, k // 16])).item())
    return q * s


def test_gemm_matches_exact_rational_triple_loop():
    rng = np.random.default_rng(0)
    for (M, N, K) in [(3, 5, 16), (4, 2, 48), (1, 1, 64)]:
        ac, asc = _rand_operand(rng, M, K, 0x00, 0xFF)
        bc, bsc = _rand_operand(rng, N, K, 0x00, 0xFF)
        tsa, tsb = np.float32(0.37), np.float32(1.5e-3)
        C, bound = gemm.gemm_nt(ac, asc, tsa, bc, bsc, tsb)
        for i in range(M):
            for j in range(N):
                exact = sum(_exact_value(ac, asc, i, k) * _exact_value(bc, bsc, j, k)
                            for k in range(K))
                exact *= Fraction(float(tsa)) * Fraction(float(tsb))
                absum = sum(abs(_exact_value(ac, asc, i, k) * _exact_value(bc, bsc, j, k))
                            for k in range(K)) * abs(Fraction(float(tsa)) * Fraction(float(tsb)))
                assert abs(Fraction(C[i, j]) - exact) <= Fraction(K * 2 ** -52) * absum + 0
                assert abs(Fraction(bound[i, j]) - absum) <= Fraction(K * 2 ** -52) * absum


def test_gemm_integer_special_case():
    """ts = 1 and every scale 1.0 (0x78): 2q is an integer, so the product is
    (2A)(2B)^T / 4 computed exactly with int64."""
    rng = np.random.default_rng(1)
    M, N, K = 33, 17, 160
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    asc = np.full((M, K // 16), 0x78, np.uint8)
    bsc = np.full((N, K // 16), 0x78, np.uint8)
    C, _ = gemm.gemm_nt(ac, asc, 1.0, bc, bsc, 1.0)
    A2 = np.rint(2 * formats.e2m1_decode(quantize.unpack_codes(ac))).astype(np.int64)
    B2 = np.rint(2 * formats.e2m1_decode(quantize.unpack_codes(bc))).astype(np.int64)
    np.testing.assert_array_equal(C * 4, (A2 @ B2.T).astype(np.float64))


def test_flushed_block_contributes_zero():
    rng = np.random.default_rng(2)
    ac, asc = _rand_operand(rng, 8, 64)
    bc, bsc = _rand_operand(rng, 8, 64)
    asc2 = asc.copy()
    asc2[:, 1] = 0x00
    ac2 = ac.copy()
    ac2[:, 8:16] = 0
    C1, _ = gemm.gemm_nt(ac2, asc, 1.0, bc, bsc, 1.0)
    C2, _ = gemm.gemm_nt(ac, asc2, 1.0, bc, bsc, 1.0)
    np.testing.assert_array_equal(C1, C2)


def test_nan_scale_poisons_row():
    rng = np.random.default_rng(3)
    ac, asc = _rand_operand(rng, 4, 32)
    bc, bsc = _rand_operand(rng, 5, 32)
    asc[2, 0] = 0xFF
    C, _ = gemm.gemm_nt(ac, asc, 1.0, bc, bsc, 1.0)
    assert np.all(np.isnan(C[2])) and np.all(np.isfinite(np.delete(C, 2, axis=0)))


def test_sampled_entries_match_full():
    rng = np.random.default_rng(4)
    ac, asc = _rand_operand(rng, 40, 96)
    bc, bsc = _rand_operand(rng, 24, 96)
    C, bound = gemm.gemm_nt(ac, asc, 0.5, bc, bsc, 2.0)
    rows = rng.integers(0, 40, 50)
    cols = rng.integers(0, 24, 50)
    v, b = gemm.gemm_nt_entries(ac, asc, 0.5, bc, bsc, 2.0, rows, cols)
    np.testing.assert_allclose(v, C[rows, cols], rtol=0, atol=1e-12 * np.abs(bound).max())
    np.testing.assert_allclose(b, bound[rows, cols], rtol=1e-14)


def test_three_gemms_of_a_linear_layer():
    """fprop, dgrad and wgrad built from the quantized operands approximate
    X W^T, dY W and dY^T X of the bf16 inputs to within the FP4 error."""
    X = random_bf16((64, 96), seed=11)
    W = random_bf16((48, 96), seed=12)
    dY = random_bf16((64, 48), seed=13, kind="gradient")
    Xf, Wf, dYf = (formats.bf16_to_f32(t).astype(np.float64) for t in (X, W, dY))
    ts = {k: np.float32(np.max(np.abs(v)) / 43008.0) for k, v in
          (("X", Xf), ("W", Wf), ("dY", dYf))}

    def q(t, name, o, rnd=quantize.RNE):
        return quantize.quantize_blockscale(t, ts[name], rnd, seed=5, orientation=o)

    Y, _ = gemm.gemm_nt(*q(X, "X", 0), ts["X"], *q(W, "W", 0), ts["W"])
    dX, _ = gemm.gemm_nt(*q(dY, "dY", 0, quantize.SR), ts["dY"], *q(W, "W", 1), ts["W"])
    dW, _ = gemm.gemm_nt(*q(dY, "dY", 1, quantize.SR), ts["dY"], *q(X, "X", 1), ts["X"])
    for got, ref in ((Y, Xf @ Wf.T), (dX, dYf @ Wf), (dW, dYf.T @ Xf)):
        assert got.shape == ref.shape
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < 0.2, rel  # E2M1 has one mantissa bit: ~10% element error

"""Pins of the MXFP4 comparison-GEMM oracle (OCP Microscaling: E2M1 elements,
one E8M0 scale per 32 elements; "format-aware fusion" article on the UFP4
page: the MXFP4 route of native FP4 hardware)."""

from fractions import Fraction

import numpy as np

from oracle import formats, mxfp4, quantize


def test_e8m0_decode_matches_fp32_exponent_field():
    """2^(c-127) is the fp32 whose exponent field is c and mantissa 0 (c =
    1..254); c = 0 is 2^-127 (the fp32 subnormal 0x00400000); 0xFF is NaN."""
    c = np.arange(1, 255, dtype=np.uint32)
    via_bits = (c << 23).view(np.float32).astype(np.float64)
    assert np.array_equal(mxfp4.e8m0_decode(c), via_bits)
    assert mxfp4.e8m0_decode(0) == np.array([0x00400000], dtype=np.uint32).view(np.float32)[0]
    assert mxfp4.e8m0_decode(127) == 1.0
    assert np.isnan(mxfp4.e8m0_decode(0xFF))


def _exact(codes, scales, i, k):
    byte = int(codes[i, k // 2])
    nib = byte & 0xF if k % 2 == 0 else byte >> 4
    q = Fraction(formats.e2m1_decode(nib).item())
    c = int(scales[i, k // 32])
    return q * (Fraction(2) ** (c - 127))


def test_gemm_matches_exact_rational_triple_loop():
    rng = np.random.default_rng(5)
    for (M, N, K) in [(3, 4, 32), (2, 2, 96), (1, 1, 64)]:
        ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        asc = rng.integers(100, 150, size=(M, K // 32), dtype=np.uint8)
        bsc = rng.integers(100, 150, size=(N, K // 32), dtype=np.uint8)
        tsa, tsb = np.float32(0.75), np.float32(3e-3)
        C, bound = mxfp4.gemm_nt_mx(ac, asc, tsa, bc, bsc, tsb)
        for i in range(M):
            for j in range(N):
                terms = [_exact(ac, asc, i, k) * _exact(bc, bsc, j, k) for k in range(K)]
                st = Fraction(float(tsa)) * Fraction(float(tsb))
                exact, absum = sum(terms) * st, sum(abs(t) for t in terms) * abs(st)
                assert abs(Fraction(C[i, j]) - exact) <= Fraction(K * 2 ** -52) * absum
                assert abs(Fraction(bound[i, j]) - absum) <= Fraction(K * 2 ** -52) * absum


def test_gemm_integer_special_case_and_scale_shift():
    """All scales 127 and ts = 1: 2q is an integer, so C = (2A)(2B)^T / 4 in
    int64; raising every A scale by one doubles C exactly."""
    rng = np.random.default_rng(6)
    M, N, K = 17, 9, 192
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s127a = np.full((M, K // 32), 127, np.uint8)
    s127b = np.full((N, K // 32), 127, np.uint8)
    C, _ = mxfp4.gemm_nt_mx(ac, s127a, 1.0, bc, s127b, 1.0)
    A2 = np.rint(2 * formats.e2m1_decode(quantize.unpack_codes(ac))).astype(np.int64)
    B2 = np.rint(2 * formats.e2m1_decode(quantize.unpack_codes(bc))).astype(np.int64)
    assert np.array_equal(C * 4, (A2 @ B2.T).astype(np.float64))
    C2, _ = mxfp4.gemm_nt_mx(ac, s127a + 1, 1.0, bc, s127b, 1.0)
    assert np.array_equal(C2, 2 * C)


def test_nan_scale_poisons_its_row_only():
    rng = np.random.default_rng(7)
    ac = rng.integers(0, 256, size=(4, 32), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)
    asc = np.full((4, 2), 127, np.uint8)
    bsc = np.full((3, 2), 127, np.uint8)
    asc[2, 1] = 0xFF
    C, _ = mxfp4.gemm_nt_mx(ac, asc, 1.0, bc, bsc, 1.0)
    assert np.all(np.isnan(C[2])) and not np.any(np.isnan(np.delete(C, 2, axis=0)))

"""Pins of the oracle's 2-D (16 x 16 tile) quantizer.

[TIBQ] summary in the UE5M3 paper's related-papers list: 2-D blocks give the
same scale to a value in the forward and in the backward (transposed) GEMM
operand.  The reading of the arithmetic is stated in oracle/quantize2d.py.

The pins reach the 2-D result by other routes than its own definition:
  - the 1-D quantizer (pinned on its own) on tensors where every 16-element
    row and column segment of a tile holds the tile's largest magnitude, so
    1-D and 2-D blocks get the same scale;
  - monotonicity of the UE5M3 encoder: the tile code is the largest of the
    16 row-block codes of the 1-D quantizer, and of the 16 column-block codes;
  - transposition invariance, and exact round trips of worked tiles.
"""

import numpy as np
import pytest

from oracle import formats, quantize, quantize2d
from workloads import random_bf16, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _diagonal_max(xb, seed):
    """Copy of xb (bf16 bits) in which every tile holds its largest magnitude
    on a permuted diagonal (random signs): then every row and every column of
    the tile contains the tile amax."""
    rng = np.random.default_rng(seed)
    x = formats.bf16_to_f32(xb).copy()
    R, C = x.shape
    for I in range(R // 16):
        for J in range(C // 16):
            t = x[16 * I:16 * I + 16, 16 * J:16 * J + 16]
            m = np.max(np.abs(t))
            perm = rng.permutation(16)
            sgn = np.where(rng.random(16) < 0.5, -1.0, 1.0).astype(np.float32)
            t[np.arange(16), perm] = sgn * m
    out = to_bf16_bits(x)
    assert np.array_equal(formats.bf16_to_f32(out), x)
    return out


@pytest.mark.parametrize("kind", ["normal", "heavy", "logrange"])
@pytest.mark.parametrize("rounding", [quantize.RNE, quantize.SR])
def test_reduces_to_1d_when_rows_and_columns_share_the_tile_amax(kind, rounding):
    xb = _diagonal_max(random_bf16((48, 64), 11, kind), 5)
    ts = np.float32(quantize.tensor_amax(xb) / np.float32(43008.0))
    rc, rs, cc, cs, _ = quantize2d.quantize_blockscale_2d(xb, ts, rounding, seed=77, offset=3)
    c1, s1 = quantize.quantize_blockscale(xb, ts, rounding, seed=77, offset=3, orientation=0)
    np.testing.assert_array_equal(rc, c1)
    np.testing.assert_array_equal(rs, s1)
    # the transposed output carries the row-wise codes (same element, same draw)
    codes = quantize.unpack_codes(c1)
    np.testing.assert_array_equal(quantize.unpack_codes(cc), codes.T)
    if rounding == quantize.RNE:
        # and, rounding to nearest, equals the 1-D quantization of x^T
        c1t, s1t = quantize.quantize_blockscale(xb, ts, rounding, orientation=1)
        np.testing.assert_array_equal(cc, c1t)
        np.testing.assert_array_equal(cs, s1t)


@pytest.mark.parametrize("kind", ["normal", "heavy", "logrange"])
def test_tile_code_is_max_of_1d_block_codes(kind):
    xb = random_bf16((64, 96), 21, kind)
    x = formats.bf16_to_f32(xb).copy()
    x[16:32, 32:48] = 0.0          # an all-zero tile -> code 0
    x[40, 70] = np.nan            # a NaN tile -> 0xFF
    x[0:16, 80:96] *= 1e-30       # tiny tile (flushes or subnormal scale)
    xb = to_bf16_bits(x)
    for ts in (np.float32(1e-3), np.float32(0.37), np.float32(2.0 ** -20)):
        t = quantize2d.tile_codes(xb, ts)
        _, s_row = quantize.quantize_blockscale(xb, ts, quantize.RNE, orientation=0)
        _, s_col = quantize.quantize_blockscale(xb, ts, quantize.RNE, orientation=1)
        R, C = x.shape
        from_rows = s_row.reshape(R // 16, 16, C // 16).max(axis=1)
        from_cols = s_col.reshape(C // 16, 16, R // 16).max(axis=1).T
        np.testing.assert_array_equal(t, from_rows)
        np.testing.assert_array_equal(t, from_cols)
    assert quantize2d.tile_codes(xb, np.float32(1e-3))[1, 2] == 0
    assert quantize2d.tile_codes(xb, np.float32(1e-3))[2, 4] == 0xFF


@pytest.mark.parametrize("kind", ["normal", "heavy", "gradient"])
def test_transposition_invariance(kind):
    xb = random_bf16((32, 80), 31, kind)
    ts = np.float32(quantize.tensor_amax(xb) / np.float32(43008.0))
    a = quantize2d.quantize_blockscale_2d(xb, ts, quantize.RNE)
    b = quantize2d.quantize_blockscale_2d(np.ascontiguousarray(xb.T), ts, quantize.RNE)
    np.testing.assert_array_equal(a[0], b[2])
    np.testing.assert_array_equal(a[1], b[3])
    np.testing.assert_array_equal(a[2], b[0])
    np.testing.assert_array_equal(a[3], b[1])
    np.testing.assert_array_equal(a[4], b[4].T)


def test_worked_tiles_round_trip_exactly():
    """ts = 1; tile (0, J) = s_J * g with s_J a normal UE5M3 value and g signed
    grid values holding 6 once: the tile code is s_J's and both outputs
    dequantize to x exactly."""
    rng = np.random.default_rng(4)
    codes_s = np.arange(0x08, 0xFF, 4)
    n = codes_s.size
    g_codes = rng.integers(0, 16, size=(16, 16 * n)).astype(np.uint8)
    g_codes[g_codes % 8 == 7] = 6    # no +-6 except the one placed below
    for J in range(n):
        g_codes[rng.integers(0, 16), 16 * J + rng.integers(0, 16)] = 7 + 8 * (J % 2)
    s = np.repeat(formats.ue5m3_decode(codes_s), 16)
    x = (formats.e2m1_decode(g_codes) * s[None, :]).astype(np.float32)
    xb = to_bf16_bits(x)
    assert np.array_equal(formats.bf16_to_f32(xb), x)
    rc, rs, cc, cs, t = quantize2d.quantize_blockscale_2d(xb, 1.0, quantize.RNE)
    np.testing.assert_array_equal(t[0], codes_s)
    np.testing.assert_array_equal(quantize.unpack_codes(rc), g_codes)
    np.testing.assert_array_equal(quantize.dequantize(rc, rs, 1.0), x)
    np.testing.assert_array_equal(quantize.dequantize(cc, cs, 1.0), x.T)


def test_sr_bits_are_the_row_orientation_stream():
    """Stochastic rounding draws element (i, j)'s bits from the row-wise
    counter: with every tile amax the same in 1-D and 2-D, SR codes of both
    outputs equal the 1-D row-wise SR codes (and differ from the 1-D
    transposed quantization, which draws from the other orientation)."""
    xb = _diagonal_max(random_bf16((32, 32), 41, "gradient"), 6)
    ts = np.float32(quantize.tensor_amax(xb) / np.float32(43008.0))
    _, _, cc, _, _ = quantize2d.quantize_blockscale_2d(xb, ts, quantize.SR, seed=9, offset=1)
    c1, _ = quantize.quantize_blockscale(xb, ts, quantize.SR, seed=9, offset=1, orientation=0)
    c1t, _ = quantize.quantize_blockscale(xb, ts, quantize.SR, seed=9, offset=1, orientation=1)
    np.testing.assert_array_equal(quantize.unpack_codes(cc), quantize.unpack_codes(c1).T)
    assert not np.array_equal(cc, c1t)


def test_rne_error_bound():
    """|dequant - x| is at most half an E2M1 step at |v| (times ts s_t), and
    the largest element of a tile clips by at most 2^-4 relative."""
    xb = random_bf16((64, 64), 51, "heavy")
    x = formats.bf16_to_f32(xb).astype(np.float64)
    ts = np.float32(quantize.tensor_amax(xb) / np.float32(43008.0))
    rc, rs, _, _, _ = quantize2d.quantize_blockscale_2d(xb, ts, quantize.RNE)
    unit = formats.ue5m3_decode(rs).astype(np.float64).repeat(16, axis=1) * float(ts)
    v = np.abs(x) / unit
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    err = np.abs(quantize.dequantize(rc, rs, ts).astype(np.float64) - x) / unit
    clip = np.maximum(v - 6.0, 0.0)
    assert np.all(err <= np.maximum(half, clip) * (1 + 1e-6) + 1e-6)
    assert np.all(clip <= 6.0 * 2.0 ** -4 + 1e-6)


def test_shape_validation():
    with pytest.raises(ValueError):
        quantize2d.tile_codes(np.zeros((16, 24), dtype=np.uint16), 1.0)
    with pytest.raises(ValueError):
        quantize2d.tile_codes(np.zeros((8, 16), dtype=np.uint16), 1.0)


def test_row_slice_matches_full():
    """A 16-aligned slice of rows (row0) reproduces those rows of the whole
    tensor's result, stochastic bits included."""
    xb = random_bf16((96, 48), 61, "gradient")
    ts = np.float32(quantize.tensor_amax(xb) / np.float32(43008.0))
    full = quantize2d.quantize_blockscale_2d(xb, ts, quantize.SR, seed=3, offset=4)
    part = quantize2d.quantize_blockscale_2d(xb[32:64], ts, quantize.SR, seed=3, offset=4, row0=32)
    np.testing.assert_array_equal(part[0], full[0][32:64])
    np.testing.assert_array_equal(part[1], full[1][32:64])
    np.testing.assert_array_equal(part[2], full[2][:, 16:32])

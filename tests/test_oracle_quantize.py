"""Pins of the oracle's block-16 quantizer (worked blocks, special cases, invariants).

[UE5M3] abstract: E2M1 payloads with UE5M3 scales per 16-element block under a
tensor scale; [TIBQ] summary: the transposed operand is quantized along its own
axis.  The arithmetic reading is stated in oracle/quantize.py.
"""

import numpy as np
import pytest

from oracle import formats, quantize, tensor_scale
from workloads import random_bf16, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _pack(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_worked_blocks_every_normal_scale():
    """ts = 1, block = s * g for every normal UE5M3 value s and a pattern g of
    signed grid values containing +-6: the scale code is s's code and every
    payload code is g's code (s * g is exact in bf16)."""
    rng = np.random.default_rng(3)
    codes_s = np.arange(0x08, 0xFF)
    s = formats.ue5m3_decode(codes_s)
    g_codes = rng.integers(0, 16, size=(codes_s.size, 16)).astype(np.uint8)
    g_codes[:, rng.integers(0, 16)] = 7  # one element at +6 fixes amax = 6 s
    g_codes[::2, 3] = 15  # some blocks also hold -6
    g = formats.e2m1_decode(g_codes)
    x = (g * s[:, None]).astype(np.float32)
    xb = to_bf16_bits(x)
    assert np.array_equal(formats.bf16_to_f32(xb), x)  # exact in bf16
    c, sc = quantize.quantize_blockscale(xb, 1.0, quantize.RNE)
    np.testing.assert_array_equal(sc[:, 0], codes_s)
    np.testing.assert_array_equal(c, _pack(g_codes))
    # and dequantization reproduces x exactly
    np.testing.assert_array_equal(quantize.dequantize(c, sc, 1.0), x)


def test_worked_block_by_hand():
    """One block worked by hand.  x = [3, -1.2, 0.1, 0, ...], ts = 0.5:
    K = 3, amax = 3, s_raw = 1 -> code 0x78 (s_b = 1), d = 0.5, r = 2,
    v = [6, -2.4, 0.2, 0] -> codes [7, 8|4, 0, 0] (2.4 rounds to 2, 0.2 to 0)."""
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :3] = [3.0, -1.2, 0.1]
    c, s = quantize.quantize_blockscale(to_bf16_bits(x), 0.5, quantize.RNE)
    assert s.tolist() == [[0x78]]
    expect = [7, 0xC, 0, 0] + [0] * 12
    assert c.tolist() == _pack([expect]).tolist()


def test_zero_and_negative_zero_block():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 16:] = -0.0
    c, s = quantize.quantize_blockscale(to_bf16_bits(x), 1.0, quantize.RNE)
    assert s.tolist() == [[0, 0]]
    assert c[0, :8].tolist() == [0] * 8
    assert c[0, 8:].tolist() == [0x88] * 8  # sign bits kept


def test_saturating_scale_and_clipping():
    """A block whose raw scale exceeds the largest UE5M3 value gets 0xFE and its
    elements saturate at 6; a raw scale that rounds down clips the block max
    to 6 as well."""
    x = np.full((1, 16), 1.0e6, dtype=np.float32)
    c, s = quantize.quantize_blockscale(to_bf16_bits(x), 1.0, quantize.RNE)
    assert s[0, 0] == 0xFE and np.all(c == 0x77)
    # s_raw = 1.0625 * 2^k rounds down to 1.0 * 2^k, so v(max) = 6.375 -> 6
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = 6.375
    c, s = quantize.quantize_blockscale(to_bf16_bits(x), 1.0, quantize.RNE)
    assert s[0, 0] == 0x78 and (c[0, 0] & 0xF) == 7


def test_subnormal_and_flushed_scales():
    x = np.zeros((1, 48), dtype=np.float32)
    x[0, 0] = 6 * 2.0 ** -17      # s_raw = 2^-17  -> 0x01
    x[0, 16] = 6 * 2.0 ** -16     # s_raw = 2^-16  -> 0x02
    x[0, 32] = 6 * 2.0 ** -19     # s_raw = 2^-19 -> 0x00 (flushed)
    c, s = quantize.quantize_blockscale(to_bf16_bits(x), 1.0, quantize.RNE)
    assert s.tolist() == [[0x01, 0x02, 0x00]]
    assert c[0, 0] & 0xF == 7 and c[0, 8] & 0xF == 7 and c[0, 16] == 0


def test_nonfinite_inputs_give_nan_blocks():
    x = np.ones((2, 32), dtype=np.float32)
    x[0, 3] = np.inf
    x[1, 20] = np.nan
    xb = to_bf16_bits(x)
    c, s = quantize.quantize_blockscale(xb, 1.0, quantize.RNE)
    assert s[0, 0] == 0xFF and s[1, 1] == 0xFF
    # magnitudes are 0 (only sign bits may remain; a NaN keeps its sign bit too)
    assert np.all((c[0, :8] & 0x77) == 0) and np.all((c[1, 8:] & 0x77) == 0)
    assert np.all(c[0, :8] == 0)  # +1 and +inf: positive
    deq = quantize.dequantize(c, s, 1.0)
    assert np.all(np.isnan(deq[0, :16])) and np.all(np.isfinite(deq[0, 16:]))
    assert np.isnan(quantize.tensor_amax(xb))


def test_degenerate_tensor_scales():
    """ts = 0 gives K = 0, s_raw = inf or NaN -> every block 0xFF; ts = inf
    gives s_raw = 0 -> every block flushed."""
    xb = random_bf16((4, 32), seed=1)
    _, s = quantize.quantize_blockscale(xb, 0.0, quantize.RNE)
    assert np.all(s == 0xFF)
    c, s = quantize.quantize_blockscale(xb, np.inf, quantize.RNE)
    assert np.all(s == 0x00) and np.all((c & 0x77) == 0)


def test_transposed_output_is_quantization_of_transpose():
    xb = random_bf16((64, 48), seed=2, kind="heavy")
    c1, s1 = quantize.quantize_blockscale(xb, 0.01, quantize.RNE, orientation=1)
    c0, s0 = quantize.quantize_blockscale(np.ascontiguousarray(xb.T), 0.01, quantize.RNE)
    assert c1.shape == (48, 32) and s1.shape == (48, 4)
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(s1, s0)
    # SR: the scales are rounded to nearest, so they match too; the payloads
    # use a different random stream (orientation 1) but stay within one step.
    cs, ss = quantize.quantize_blockscale(xb, 0.01, quantize.SR, seed=9, orientation=1)
    np.testing.assert_array_equal(ss, s1)
    dq_sr = quantize.dequantize_unscaled(cs, ss)
    dq_rne = quantize.dequantize_unscaled(c1, s1)
    s_b = np.repeat(formats.ue5m3_decode(ss), 16, axis=1)
    assert np.all(np.abs(dq_sr - dq_rne) <= 2 * s_b + 0)


def test_row_subset_matches_full():
    xb = random_bf16((96, 64), seed=4, kind="gradient")
    ts = np.float32(1e-7)
    for rounding in (quantize.RNE, quantize.SR):
        for o in (0, 1):
            cf, sf = quantize.quantize_blockscale(xb, ts, rounding, seed=3, offset=2, orientation=o)
            rows = [0, 5, cf.shape[0] - 1, 17]
            cs, ss = quantize.quantize_blockscale(xb, ts, rounding, seed=3, offset=2,
                                                  orientation=o, rows=rows)
            np.testing.assert_array_equal(cs, cf[rows])
            np.testing.assert_array_equal(ss, sf[rows])


def test_rne_error_bound():
    """Round-to-nearest error of every unsaturated element is at most half a
    grid step times ts * s_b; saturated elements are those with |v| > 6."""
    xb = random_bf16((256, 256), seed=5)
    x = formats.bf16_to_f32(xb).astype(np.float64)
    ts = np.float32(np.max(np.abs(x)) / (6 * 7168.0))
    c, s = quantize.quantize_blockscale(xb, ts, quantize.RNE)
    deq = quantize.dequantize_unscaled(c, s) * float(ts)
    sb = np.repeat(formats.ue5m3_decode(s), 16, axis=1) * float(ts)
    v = np.abs(x) / sb
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    ok = v <= 6
    err = np.abs(deq - x)
    assert np.all(err[ok] <= 0.5 * step[ok] * sb[ok] * (1 + 2 ** -20))
    # the block scale is within half a UE5M3 step of amax_b / (6 ts)
    amax_b = np.abs(x).reshape(256, 16, 16).max(axis=2)
    s_raw = amax_b / (6 * float(ts))
    rel = np.abs(formats.ue5m3_decode(s) - s_raw) / s_raw
    assert np.all(rel <= 1 / 16 + 1e-6)


def test_tensor_amax():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((128, 64)).astype(np.float32) * 0.1
    x[77, 13] = -9.5
    assert quantize.tensor_amax(to_bf16_bits(x)) == np.float32(9.5)
    assert quantize.tensor_amax(np.zeros((0, 16), np.uint16)) == 0


def test_stale_scale_absorbed_without_saturation():
    """Dynamic-range stress: block magnitudes log-uniform over 2^-24..2^12 and
    a tensor scale from an amax that is off by x8 or x1/8.  With max_safe =
    7168 no block saturates (raw scale > 114688) in either case."""
    from workloads import log_uniform_blocks

    rng = np.random.default_rng(10)
    xb = to_bf16_bits(log_uniform_blocks(rng, (512, 512)))
    amax = quantize.tensor_amax(xb)
    x = formats.bf16_to_f32(xb)
    amax_b = np.abs(x).reshape(512, 32, 16).max(axis=2)
    for factor in (8.0, 0.125):
        _, ts = tensor_scale.update_tensor_scale(np.float32(amax * factor), 1.0, 0, 1)
        c, s = quantize.quantize_blockscale(xb, ts, quantize.RNE)
        s_raw = amax_b / (np.float32(6) * ts)
        assert np.all(s_raw <= formats.UE5M3_MAX)
        assert not np.any(s == 0xFF)
        flushed = np.mean((s == 0) & (amax_b > 0))
        assert flushed < 0.35


def test_shapes_and_validation():
    xb = random_bf16((32, 48), seed=8)
    c, s = quantize.quantize_blockscale(xb, 1.0)
    assert c.shape == (32, 24) and s.shape == (32, 3)
    c, s = quantize.quantize_blockscale(xb, 1.0, orientation=1)
    assert c.shape == (48, 16) and s.shape == (48, 2)
    with pytest.raises(ValueError):
        quantize.quantize_blockscale(random_bf16((32, 40), seed=8), 1.0)

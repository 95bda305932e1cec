"""Pins of the oracle's stochastic rounding (SR) for backward gradients.

[UE5M3] abstract: selective stochastic rounding on backward gradients; [UFP4]
abstract: stochastic rounding restricted to dY.  Stochastic rounding must be
unbiased: the expected rounded value equals the input.  With 16 random bits
the oracle rounds up with probability ceil(65536 * frac) / 65536 (frac = the
position of the value between its two grid neighbours), so the bias is at
most one grid step * 2^-16.
"""

import math

import numpy as np

from oracle import formats, quantize

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_sr_exact_probability_all_random_values():
    """For each probe, enumerate all 65536 random values: the number that round
    up must be exactly ceil(65536 * frac) (closed form)."""
    u = np.arange(65536, dtype=np.uint16)
    probes = [0.1, 0.25, 0.3, 0.5, 0.7, 1.0 + 2 ** -20, 1.2, 1.75, 1.9, 2.0, 2.3,
              2.5, 3.999, 4.0 + 2 ** -21, 4.5, 5.0, 5.9, 5.9999995]
    for p in probes:
        a = np.float32(p)
        idx = formats.e2m1_round_stochastic(np.full(65536, a), u)
        lo_i = max(i for i, g in enumerate(GRID) if g <= float(a))
        lo, hi = GRID[lo_i], GRID[lo_i + 1]
        frac = (float(a) - lo) / (hi - lo)
        n_up = int(np.sum(idx == lo_i + 1))
        assert np.all((idx == lo_i) | (idx == lo_i + 1)), p
        assert n_up == math.ceil(65536 * frac), (p, n_up, frac)


def test_sr_grid_values_and_saturation_are_deterministic():
    u = np.arange(0, 65536, 97, dtype=np.uint16)
    for i, g in enumerate(GRID):
        idx = formats.e2m1_round_stochastic(np.full(u.size, np.float32(g)), u)
        assert np.all(idx == i)
    for big in (6.0, 6.1, 100.0, np.inf):
        idx = formats.e2m1_round_stochastic(np.full(u.size, np.float32(big)), u)
        assert np.all(idx == 7)


def _constant_blocks(x, rows=4096, cols=32):
    """bf16 tensor whose 16-blocks are [6, x, x, ..., x]: with ts = 1 the block
    scale is exactly 1 (0x78) and the scaled value of every x is x itself."""
    from workloads import to_bf16_bits

    t = np.full((rows, cols), x, dtype=np.float32)
    t[:, 0::16] = 6.0
    return to_bf16_bits(t)


def test_sr_unbiased_over_1e5_seeded_draws():
    """Mean of >= 1e5 stochastically rounded copies of one value is within
    1e-3 relative of the value (and within 5 standard errors)."""
    for p in (1.9, 5.9, 2.7, 4.6, 1.3, 3.2):
        xb = _constant_blocks(p)
        x = float(formats.bf16_to_f32(xb[0, 1]))
        codes, scales = quantize.quantize_blockscale(xb, 1.0, quantize.SR, seed=1234, offset=5)
        assert np.all(scales == 0x78)
        deq = quantize.dequantize(codes, scales, 1.0)
        mask = np.ones(xb.shape, dtype=bool)
        mask[:, 0::16] = False
        vals = deq[mask].astype(np.float64)
        assert vals.size >= 100000
        lo = max(g for g in GRID if g <= x)
        hi = min(g for g in GRID if g > x)
        frac = (x - lo) / (hi - lo)
        sigma = (hi - lo) * math.sqrt(frac * (1 - frac)) / math.sqrt(vals.size)
        err = vals.mean() - x
        assert abs(err) / x < 1e-3, (p, err / x)
        assert abs(err) < 5 * sigma + (hi - lo) * 2 ** -16, (p, err, sigma)
        assert set(np.unique(vals)) <= {lo, hi}


def test_sr_whole_tensor_mean():
    """Over a gradient-like tensor the SR dequantization error averages out;
    round-to-nearest leaves the E2M1 grid's systematic error."""
    from workloads import random_bf16

    xb = random_bf16((1024, 256), seed=21, kind="gradient")
    x = formats.bf16_to_f32(xb).astype(np.float64)
    amax = float(np.max(np.abs(x)))
    ts = np.float32(amax / (6 * 7168.0))
    c, s = quantize.quantize_blockscale(xb, ts, quantize.SR, seed=77, offset=1)
    err = quantize.dequantize(c, s, ts).astype(np.float64) - x
    # mean signed error relative to mean |x|: zero-mean noise of size ~1/sqrt(n)
    rel = abs(err.mean()) / np.abs(x).mean()
    assert rel < 5e-3, rel
    # per-element error of SR is below one grid step: |err| < step * ts * s_b
    c2, s2 = quantize.quantize_blockscale(xb, ts, quantize.RNE)
    err_rne = quantize.dequantize(c2, s2, ts).astype(np.float64) - x
    assert np.abs(err).max() <= 2.1 * np.abs(err_rne).max() + 1e-30


def test_sr_random_bits_differ_by_seed_and_offset():
    xb = _constant_blocks(1.9, rows=64)
    a = quantize.quantize_blockscale(xb, 1.0, quantize.SR, seed=1, offset=0)[0]
    b = quantize.quantize_blockscale(xb, 1.0, quantize.SR, seed=2, offset=0)[0]
    c = quantize.quantize_blockscale(xb, 1.0, quantize.SR, seed=1, offset=1)[0]
    a2 = quantize.quantize_blockscale(xb, 1.0, quantize.SR, seed=1, offset=0)[0]
    assert np.array_equal(a, a2)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)

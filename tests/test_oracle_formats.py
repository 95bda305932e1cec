"""Pins of the oracle's E2M1 and UE5M3 formats against facts fixed outside it.

Sources: [UE5M3] "UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", abstract (E2M1 payloads, unsigned E5M3 block scales).  The bit
layouts are readings stated in oracle/formats.py; these tests pin the oracle's
code to them by routes that do not reuse its formulas: the listed E2M1
magnitudes, numpy's IEEE binary16 decoder, hand-derived rounding thresholds
and exact integer nearest-value searches.
"""

import numpy as np

from oracle import formats

E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ------------------------------------------------------------------ E2M1 --

def test_e2m1_decode_table():
    vals = formats.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == E2M1_MAGNITUDES
    assert list(-vals[8:]) == E2M1_MAGNITUDES
    assert np.signbit(vals[8])  # code 8 is -0


def test_e2m1_every_magnitude_round_trips():
    for idx, mag in enumerate(E2M1_MAGNITUDES):
        a = np.array([mag], dtype=np.float32)
        assert formats.e2m1_round_nearest_even(a)[0] == idx
        # stochastic rounding of an exact grid value never moves it
        for u in (0, 1, 32768, 65535):
            assert formats.e2m1_round_stochastic(a, np.array([u], np.uint16))[0] == idx


# Hand-derived round-to-nearest-even thresholds on the grid 0 .5 1 1.5 2 3 4 6:
# (midpoint, index just below it, index just above it, index AT the midpoint).
# At a midpoint the even index wins.
RNE_MIDPOINTS = [
    (0.25, 0, 1, 0),
    (0.75, 1, 2, 2),
    (1.25, 2, 3, 2),
    (1.75, 3, 4, 4),
    (2.5, 4, 5, 4),
    (3.5, 5, 6, 6),
    (5.0, 6, 7, 6),
]


def _threshold_rne(a):
    """Independent formulation: count the thresholds that a has passed."""
    a = a.astype(np.float64)
    idx = np.zeros(a.shape, dtype=np.int64)
    for mid, _below, above, at in RNE_MIDPOINTS:
        # a value exactly at the midpoint goes to `at`
        passed = (a > mid) | ((a == mid) & (at == above))
        idx += passed
    idx = np.where(a >= 6.0, 7, idx)
    return idx


def test_e2m1_rne_midpoints_exact():
    for mid, below, above, at in RNE_MIDPOINTS:
        m = np.float32(mid)
        lo = np.nextafter(m, np.float32(0))
        hi = np.nextafter(m, np.float32(10))
        got = formats.e2m1_round_nearest_even(np.array([lo, m, hi], dtype=np.float32))
        assert list(got) == [below, at, above], (mid, got)
        assert at % 2 == 0


def _all_f32_near(values, radius):
    bits = np.array(values, dtype=np.float32).view(np.uint32).astype(np.int64)
    offs = np.arange(-radius, radius + 1, dtype=np.int64)
    allbits = (bits[:, None] + offs[None, :]).ravel()
    allbits = allbits[(allbits >= 0) & (allbits < 0x7F800000)]
    return np.unique(allbits).astype(np.uint32).view(np.float32)


def test_e2m1_rne_brute_force():
    """Every fp32 within 4096 ulps of each midpoint and grid value, every fp32
    in [0, 8) whose low 12 mantissa bits are zero or all ones, and 2^22 random
    fp32 patterns below 8, against the threshold formulation."""
    near = _all_f32_near([m for m, *_ in RNE_MIDPOINTS] + E2M1_MAGNITUDES[1:], 4096)
    top = np.arange(0, 0x41000000 >> 12, dtype=np.uint32) << np.uint32(12)
    coarse = np.concatenate([top, top | np.uint32(0xFFF)]).view(np.float32)
    rng = np.random.default_rng(11)
    rnd = rng.integers(0, 0x41000000, size=1 << 22, dtype=np.uint32).view(np.float32)
    for a in (near, coarse, rnd):
        for start in range(0, a.size, 1 << 20):
            chunk = a[start:start + (1 << 20)]
            np.testing.assert_array_equal(formats.e2m1_round_nearest_even(chunk),
                                          _threshold_rne(chunk))


def test_e2m1_rne_saturation_and_specials():
    a = np.array([6.0, 6.5, 7.0, 1e30, np.inf, np.float32(3.4e38)], dtype=np.float32)
    assert list(formats.e2m1_round_nearest_even(a)) == [7] * 6
    assert formats.e2m1_round_nearest_even(np.array([np.nan], np.float32))[0] == 0
    assert formats.e2m1_round_nearest_even(np.array([0.0, 1e-45], np.float32)).tolist() == [0, 0]


# ----------------------------------------------------------------- UE5M3 --

def test_ue5m3_decode_matches_binary16():
    """Codes 0x00..0xF7 share IEEE binary16's exponent field (5 bits, bias 15,
    subnormals at exponent 0): code c is binary16 bit pattern c << 7."""
    codes = np.arange(0xF8)
    ref = (codes.astype(np.uint16) << 7).view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(formats.ue5m3_decode(codes), ref)


def test_ue5m3_decode_top_octave_and_nan():
    for f in range(7):
        assert formats.ue5m3_decode(0xF8 + f) == (1 + f / 8) * 65536.0
    assert formats.ue5m3_decode(0xFE) == 114688.0 == formats.UE5M3_MAX
    assert np.isnan(formats.ue5m3_decode(0xFF))
    assert formats.ue5m3_decode(0x01) == 2.0 ** -17
    assert formats.ue5m3_decode(0x08) == 2.0 ** -14
    assert formats.ue5m3_decode(0x78) == 1.0


def test_ue5m3_encode_decode_round_trip_all_codes():
    codes = np.arange(0xFF)
    vals = formats.ue5m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(formats.ue5m3_encode(vals), codes)
    assert formats.ue5m3_encode(np.float32(np.nan)) == 0xFF


def test_ue5m3_decode_strictly_increasing():
    v = formats.ue5m3_decode(np.arange(0xFF))
    assert np.all(np.diff(v) > 0)


# Exact nearest-code search: every fp32 value in [2^-18, 2^17] and every UE5M3
# value is an integer multiple of 2^-41, below 2^58, so int64 holds them all.
_Q = 41


def _exact_nearest_code(s):
    s = s.astype(np.float64)
    codes = np.arange(0xFF, dtype=np.int64)
    vals = np.rint(np.ldexp(formats.ue5m3_decode(codes), _Q)).astype(np.int64)
    S = np.rint(np.ldexp(s, _Q)).astype(np.int64)
    assert np.all(np.ldexp(S.astype(np.float64), -_Q) == s)  # exact
    hi = np.clip(np.searchsorted(vals, S, side="left"), 1, 0xFE)
    lo = hi - 1
    dlo = S - vals[lo]
    dhi = vals[hi] - S
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(S >= vals[0xFE], 0xFE, pick)
    return pick


def test_ue5m3_encode_brute_force():
    """Against the exact nearest code (ties to the even code, saturating) for:
    every fp32 in [2^-18, 2^17) with the low 8 mantissa bits in a set that
    straddles every possible tie, every fp32 of three whole octaves, and 2^22
    random fp32 patterns of that range."""
    lo_bits = np.float32(2.0 ** -18).view(np.uint32)
    hi_bits = np.float32(2.0 ** 17).view(np.uint32)
    top = np.arange(lo_bits >> 8, hi_bits >> 8, dtype=np.uint32) << np.uint32(8)
    lows = np.array([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFF], dtype=np.uint32)
    sets = [(top[:, None] | lows[None, :]).ravel()]
    for e in (-15, -1, 16):  # subnormal->normal edge, middle, top octave
        b0 = np.float32(2.0 ** e).view(np.uint32)
        sets.append(np.arange(b0, b0 + (1 << 23), dtype=np.uint32))
    rng = np.random.default_rng(12)
    sets.append(rng.integers(lo_bits, hi_bits, size=1 << 22, dtype=np.uint32))
    for bits in sets:
        for start in range(0, bits.size, 1 << 21):
            s = bits[start:start + (1 << 21)].view(np.float32)
            np.testing.assert_array_equal(formats.ue5m3_encode(s), _exact_nearest_code(s))


def test_ue5m3_encode_outside_range():
    # below 2^-18 the nearest value is 0; exactly 2^-18 ties to the even code 0x00
    tiny = np.array([1e-45, 1e-30, 2.0 ** -19, 2.0 ** -18], dtype=np.float32)
    assert formats.ue5m3_encode(tiny).tolist() == [0, 0, 0, 0]
    assert formats.ue5m3_encode(np.nextafter(np.float32(2.0 ** -18), np.float32(1))) == 1
    big = np.array([2.0 ** 17, 1.8125 * 2 ** 16, 1e30, 3.4e38], dtype=np.float32)
    assert formats.ue5m3_encode(big).tolist() == [0xFE] * 4
    specials = np.array([np.inf, -np.inf, np.nan, -1.0, -1e-30], dtype=np.float32)
    assert formats.ue5m3_encode(specials).tolist() == [0xFF] * 5
    assert formats.ue5m3_encode(np.array([0.0, -0.0], np.float32)).tolist() == [0, 0]


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x0001], dtype=np.uint16)
    f = formats.bf16_to_f32(bits)
    assert f[0] == 1.0 and f[1] == -1.0 and f[2] == 0 and np.signbit(f[3])
    assert np.isinf(f[4]) and f[5] == np.float32(2.0 ** -133)


def test_f32_to_bf16_rne_worked_cases():
    """Hand-worked roundings of the 16 dropped bits: below, at and above the
    halfway point, ties to the even pattern, the carry into the exponent and
    into Inf, signs, subnormals and NaN."""
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0x3F807FFF: 0x3F80,  # just below half an ulp: down
        0x3F808000: 0x3F80,  # tie, 0x3F80 is even: down
        0x3F808001: 0x3F81,  # just above: up
        0x3F818000: 0x3F82,  # tie, 0x3F81 is odd: up to the even one
        0x3FFF8000: 0x4000,  # tie at the top of the binade: the carry bumps the exponent
        0xBFC00000: 0xBFC0,  # -1.5
        0x7F7FFFFF: 0x7F80,  # largest fp32 rounds to +Inf
        0xFF7F8000: 0xFF80,  # tie at the top, odd: -Inf
        0x7F800000: 0x7F80,  # +Inf
        0x00008000: 0x0000,  # subnormal tie to even (zero)
        0x00018000: 0x0002,  # subnormal tie, odd: up
        0x80000000: 0x8000,  # -0
    }
    x = np.array(list(cases), dtype=np.uint32).view(np.float32)
    got = formats.f32_to_bf16_rne(x)
    assert got.tolist() == list(cases.values())
    nan = formats.f32_to_bf16_rne(np.array([0x7FC00000, 0x7F800001, 0xFFA00000], np.uint32).view(np.float32))
    assert np.all((nan & 0x7F80) == 0x7F80) and np.all((nan & 0x7F) != 0)


def test_f32_to_bf16_rne_against_torch_cast():
    """A library routine: torch's CPU fp32 -> bfloat16 cast (round to nearest
    even) on random finite patterns and on every tie pattern (low half 0x8000)
    and its two neighbours."""
    import torch

    rng = np.random.default_rng(77)
    rand = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x7FFF, hi | 0x8000, hi | 0x8001])
    bits = np.concatenate([rand, ties])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.f32_to_bf16_rne(x), want)

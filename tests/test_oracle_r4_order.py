"""Pins of reading R4's operation order in the oracle's quantizer.

[UE5M3] abstract: two-level scaling, x ~= ts * s_b * q with E2M1 payloads q,
UE5M3 block scales s_b (blocks of 16) and an fp32 tensor scale ts.  The pages
fix neither the formula nor the order of its roundings; the reading taken is
(every step one IEEE fp32 operation, round to nearest even):
    K = RN(6 ts);  s_raw = RN(amax_b / K);  s_b = UE5M3(s_raw);
    d = RN(ts s_b);  r = RN(1 / d);  v = RN(x r);  q = E2M1(v).
Worked blocks built on tensor scales that are not powers of two, where the
value lands within one fp32 ulp of a rounding midpoint, so that each plausible
alternative order gives a different code:
  - scale step:   RN(RN(amax / 6) / ts), and the exact amax / (6 ts);
  - element step: RN(x / d), and the exact x / (ts s_b).
The expected codes are derived here with exact rational arithmetic
(`fractions.Fraction`) and an explicit nearest-fp32 rounding, independently of
the oracle's numpy code; each case also checks that the alternatives disagree
with it, so the case can tell the orders apart.
"""

import struct
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import quantize


def _f32_bits(q):
    return struct.unpack("<I", struct.pack("<f", float(q)))[0]


def _bits_f32(b):
    return Fr(struct.unpack("<f", struct.pack("<I", b))[0])


def _bf16(b):
    return _bits_f32(b << 16)


def rn32(q):
    """The fp32 value nearest to the positive rational q (ties to an even
    significand); q inside the normal range."""
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fr(2) ** e > q:
        e -= 1
    assert Fr(2) ** e <= q < Fr(2) ** (e + 1) and -126 <= e <= 127
    ulp = Fr(2) ** (e - 23)
    m = q / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * ulp


def ue5m3_value(c):
    e, f = c >> 3, c & 7
    return Fr(f) * Fr(2) ** -17 if e == 0 else (1 + Fr(f, 8)) * Fr(2) ** (e - 15)


def ue5m3_nearest(s):
    """Nearest of the 255 finite UE5M3 values (ties to the even code); s in
    range, so no saturation is involved."""
    best = None
    for c in range(0xFF):
        dist = abs(ue5m3_value(c) - s)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1]


E2M1_GRID = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def e2m1_nearest(a):
    """Index of the nearest E2M1 magnitude (ties to the even index)."""
    best = None
    for i, g in enumerate(E2M1_GRID):
        dist = abs(a - g)
        if best is None or dist < best[0] or (dist == best[0] and i % 2 == 0):
            best = (dist, i)
    return best[1]


def _block(amax_bf16, x_bf16):
    """A 16-element block: the amax at element 0, x at element 5, zeros."""
    b = np.zeros((1, 16), dtype=np.uint16)
    b[0, 0] = amax_bf16
    b[0, 5] = x_bf16
    return b


# (amax bf16 bits, tensor-scale fp32 bits): the scale code by R4, by the
# alternative RN(RN(amax/6)/ts), and by the exact quotient
SCALE_CASES = [
    (0x4081, 0x3FA1E1E1),  # amax 4.03125:  R4 0x70, alternative 0x71, exact 0x71
    (0x4081, 0x3F6F4DEA),  # R4 0x73, alternative 0x74
    (0x4082, 0x3F7128D0),  # amax 4.0625: R4 0x74, alternative 0x73, exact 0x73
    (0x4082, 0x3EF128D0),  # R4 0x7C, alternative 0x7B, exact 0x7B
    (0x4081, 0x3F4BDA13),  # R4 0x76, exact 0x75
]

# (x bf16, ts fp32 bits, amax bf16): the element code by R4, by RN(x / d)
# and by the exact x / (ts s_b); x / d lies within one ulp of an E2M1 midpoint
ELEMENT_CASES = [
    (0x3F82, 0x3F7FFFFF, 0x409A),  # x 1.015625, ts 1 - 2^-24, s_b 0.8125: R4 index 2 (1.0), RN(x/d) 3 (1.5)
    (0x3F82, 0x3F1745D1, 0x409B),  # midpoint 1.25: R4 2, RN(x/d) 3
    (0x3F82, 0x3EFFFFFF, 0x401A),  # midpoint 2.5:  R4 4, RN(x/d) 5
    (0x3F82, 0x3E7FFFFF, 0x3F9A),  # midpoint 5:    R4 6, RN(x/d) 7
    (0x3F81, 0x3FB77777, 0x4099),  # midpoint 1.25: R4 2, exact quotient 3
    (0x3F81, 0x3FFA2E8C, 0x4100),  # midpoint 0.75: R4 2, exact quotient 1
]


def _scale_codes(amax, ts):
    r4 = ue5m3_nearest(rn32(amax / rn32(6 * ts)))
    alt = ue5m3_nearest(rn32(rn32(amax / 6) / ts))
    exact = ue5m3_nearest(amax / (6 * ts))
    return r4, alt, exact


@pytest.mark.parametrize("amax_b,ts_b", SCALE_CASES)
def test_scale_step_order(amax_b, ts_b):
    amax, ts = _bf16(amax_b), _bits_f32(ts_b)
    r4, alt, exact = _scale_codes(amax, ts)
    assert r4 != alt or r4 != exact, "the case does not separate the orders"
    _, scales = quantize.quantize_blockscale(_block(amax_b, 0), np.float32(float(ts)), quantize.RNE)
    assert int(scales[0, 0]) == r4, f"oracle scale {scales[0, 0]:#x}, R4 {r4:#x} (alt {alt:#x}, exact {exact:#x})"


@pytest.mark.parametrize("x_b,ts_b,amax_b", ELEMENT_CASES)
def test_element_step_order(x_b, ts_b, amax_b):
    x, ts, amax = _bf16(x_b), _bits_f32(ts_b), _bf16(amax_b)
    code = _scale_codes(amax, ts)[0]
    s_b = ue5m3_value(code)
    d = rn32(ts * s_b)
    r4 = e2m1_nearest(rn32(x * rn32(1 / d)))
    div_d = e2m1_nearest(rn32(x / d))
    exact = e2m1_nearest(x / (ts * s_b))
    assert r4 != div_d or r4 != exact, "the case does not separate the orders"
    # the block's largest element sits on the grid's top value, so the scale
    # is the one the element sees
    codes, scales = quantize.quantize_blockscale(_block(amax_b, x_b), np.float32(float(ts)), quantize.RNE)
    assert int(scales[0, 0]) == code
    got = (int(codes[0, 2]) >> 4) & 0xF  # element 5: high nibble of byte 2
    assert got == r4, f"oracle index {got}, R4 {r4} (RN(x/d) {div_d}, exact {exact})"


def test_cases_cover_both_alternatives():
    """Every alternative order is contradicted by at least one case."""
    sc = [_scale_codes(_bf16(a), _bits_f32(t)) for a, t in SCALE_CASES]
    assert any(r != a for r, a, _ in sc) and any(r != e for r, _, e in sc)
    el = []
    for x_b, ts_b, amax_b in ELEMENT_CASES:
        x, ts, amax = _bf16(x_b), _bits_f32(ts_b), _bf16(amax_b)
        s_b = ue5m3_value(_scale_codes(amax, ts)[0])
        d = rn32(ts * s_b)
        el.append((e2m1_nearest(rn32(x * rn32(1 / d))), e2m1_nearest(rn32(x / d)),
                   e2m1_nearest(x / (ts * s_b))))
    assert any(r != a for r, a, _ in el) and any(r != e for r, _, e in el)


def test_rn32_against_numpy_cast():
    """The nearest-fp32 helper agrees with numpy's float64 -> float32 cast on
    doubles (exact rationals), ties included."""
    rng = np.random.default_rng(0)
    vals = rng.uniform(1e-3, 1e3, 2000)
    ties = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 3.0 * (1 + 2.0 ** -23) + 3 * 2.0 ** -24])
    for v in np.concatenate([vals, ties]):
        assert rn32(Fr(float(v))) == Fr(float(np.float32(v)))

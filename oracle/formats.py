"""E2M1 payload and UE5M3 block-scale number formats (oracle side).

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

[UE5M3] abstract: payloads are E2M1 (4-bit floats with a narrow range of
magnitudes) and each block carries an *unsigned* E5M3 scale.  The pages give
the format names only.  Readings taken here:

E2M1 (one nibble).  Bit 3 = sign, bits 2..1 = exponent (bias 1), bit 0 =
  mantissa; no Inf or NaN.  Exponent field 0 is subnormal (0 or 0.5).  The
  eight magnitudes are therefore 0, 0.5, 1, 1.5, 2, 3, 4, 6.

UE5M3 (one byte, unsigned).  Bits 7..3 = exponent e (bias 15, as the 5-bit
  exponent of IEEE binary16), bits 2..0 = mantissa f.
    e == 0           subnormal: f * 2^-17
    0 < e, c != 0xFF (1 + f/8) * 2^(e-15)
    c == 0xFF        NaN (the only special code; there is no infinity)
  So 0x01 = 2^-17 (smallest), 0x08 = 2^-14 (smallest normal), 0x78 = 1.0 and
  0xFE = 1.75 * 2^16 = 114688 (largest).  Encoding rounds to nearest, ties to
  the even code, and saturates finite overflow to 0xFE.
"""

import numpy as np

# ---------------------------------------------------------------- E2M1 ----


def e2m1_decode(code):
    """Value of E2M1 code(s) 0..15 as float64, from the bit fields."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where((code >> 3) & 1, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    subnormal = 0.5 * m
    normal = np.ldexp(1.0 + 0.5 * m, e - 1)
    return sign * np.where(e == 0, subnormal, normal)


# Magnitudes of codes 0..7, increasing: the E2M1 grid.
E2M1_GRID = e2m1_decode(np.arange(8))
E2M1_MAX = 6.0


def e2m1_round_nearest_even(a):
    """Round magnitudes |v| (fp32 array, >= 0 or NaN) to an E2M1 magnitude index.

    Round to nearest grid value; a value exactly half-way between two grid
    values goes to the one with the even code (index).  Values >= 6 (and +Inf)
    saturate to 6 (index 7).  Reading: a NaN magnitude encodes index 0.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)  # exact
    dist = np.abs(a[..., None] - E2M1_GRID)  # exact near every tie
    best = dist.min(axis=-1, keepdims=True)
    is_min = dist == best
    even = (np.arange(8) % 2) == 0
    # At most two grid values can be equally near, and they are adjacent, so
    # exactly one of them has an even index.
    has_even = (is_min & even).any(axis=-1, keepdims=True)
    pick = np.where(has_even, is_min & even, is_min)
    idx = np.argmax(pick, axis=-1)
    idx = np.where(a >= E2M1_MAX, 7, idx)
    idx = np.where(np.isnan(a), 0, idx)
    return idx.astype(np.uint8)


def e2m1_round_stochastic(a, u16):
    """Stochastically round magnitudes |v| to an E2M1 magnitude index.

    [UE5M3] abstract: stochastic rounding is applied to backward gradients.
    Reading: let lo be the largest grid value <= a and step the distance to
    the next grid value.  The magnitude rounds up to lo + step when the 16
    random bits, read as an integer u in [0, 65535], satisfy u < frac * 65536
    with frac = (a - lo) / step; otherwise it stays at lo.  So it rounds up
    with probability ceil(65536 * frac) / 65536.  Values >= 6 saturate to 6;
    a NaN magnitude encodes index 0.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)  # exact
    u = np.asarray(u16, dtype=np.uint16).astype(np.float64)
    below = a < E2M1_MAX
    safe = np.where(below, a, 0.0)
    lo_idx = np.searchsorted(E2M1_GRID, safe, side="right") - 1
    lo_idx = np.clip(lo_idx, 0, 6)
    lo = E2M1_GRID[lo_idx]
    step = E2M1_GRID[lo_idx + 1] - lo
    frac = (safe - lo) / step  # exact: the difference and the power-of-two division
    up = u < frac * 65536.0
    idx = lo_idx + up.astype(np.int64)
    idx = np.where(below, idx, 7)
    idx = np.where(np.isnan(a), 0, idx)
    return idx.astype(np.uint8)


# --------------------------------------------------------------- UE5M3 ----

UE5M3_BIAS = 15
UE5M3_NAN = 0xFF
UE5M3_MAX_CODE = 0xFE
UE5M3_MAX = 1.75 * 2.0 ** 16  # 114688.0


def ue5m3_decode(code):
    """Value of UE5M3 code(s) 0..255 as float64 (0xFF -> NaN)."""
    code = np.asarray(code, dtype=np.int64)
    e = code >> 3
    f = code & 7
    subnormal = f * 2.0 ** -17
    normal = np.ldexp(1.0 + f / 8.0, e - UE5M3_BIAS)
    val = np.where(e == 0, subnormal, normal)
    return np.where(code == UE5M3_NAN, np.nan, val)


def ue5m3_encode(s):
    """Encode fp32 value(s) s to UE5M3, round to nearest even, saturating.

    Reading: NaN, +-Inf and negative s give 0xFF (NaN); +-0 gives 0x00.
    Otherwise, with E = max(floor(log2 s), -14), the mantissa m is s / 2^(E-3)
    rounded to the nearest integer (ties to even); m lies in [0, 16] and
    code = 8 * (E + 14) + m, capped at 0xFE.  A carry (m == 16) moves to the
    next exponent by itself, and E = -14 with m < 8 gives the subnormals.
    """
    s = np.asarray(s, dtype=np.float32).astype(np.float64)  # exact
    finite_nonneg = np.isfinite(s) & (s >= 0)
    zero = s == 0
    ok = finite_nonneg & ~zero
    t = np.where(ok, s, 1.0)
    _, ex = np.frexp(t)  # t = mant * 2^ex, mant in [0.5, 1)
    E = np.maximum(ex - 1, -14)
    m = np.rint(t / np.ldexp(1.0, E - 3))  # exact scaling; rint rounds half to even
    code = np.minimum(8 * (E + 14) + m.astype(np.int64), UE5M3_MAX_CODE)
    code = np.where(zero, 0, code)
    code = np.where(finite_nonneg, code, UE5M3_NAN)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- bf16 ----


def bf16_to_f32(bits):
    """bfloat16 bit patterns (uint16) -> float32, exactly (bits << 16)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x):
    """float32 value(s) -> bfloat16 bit patterns (uint16), round to nearest
    with ties to even on the 16 dropped bits; overflow carries into the
    exponent (to Inf); NaN stays NaN (quiet bit set).  This is the rounding of
    a GEMM output stored in bf16 (the fused-epilogue reading R19: the next
    linear quantizes bf16(C))."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (b & 0x7FFFFFFF) > 0x7F800000
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, ((b >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)

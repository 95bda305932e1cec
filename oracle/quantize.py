"""Block-16 E2M1/UE5M3 quantization under a tensor scale (oracle side).

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

[UE5M3] abstract: E2M1 payloads with unsigned E5M3 block scales, block size
16, a per-tensor scale that is refreshed periodically (not recomputed from the
current tensor before each quantization), stochastic rounding for backward
gradients only.  [TIBQ] summary: with 1-D blocks a tensor and its transpose get
different scales, so the transposed operands of the backward GEMMs are
quantized again, along their own contraction axis, from the bf16 source.

Two-level scaling, x ~= ts * s_b * q, where ts is the fp32 tensor scale, s_b
the UE5M3 scale of the 16-element block and q the E2M1 payload.

Reading for the arithmetic (every operation is one IEEE fp32 operation with
round-to-nearest-even, in this order, no fused multiply-add):
  1. x = float32(bf16 bits << 16).
  2. Blocks: 16 consecutive elements along the columns of the output
     orientation.  Orientation 0 quantizes x as given (R x C); orientation 1
     quantizes x^T (C x R): the transposed output.
  3. amax_b = max |x| over the block (a NaN propagates).
  4. K = 6 * ts once per call; s_raw = amax_b / K.  So the block's largest
     element maps onto the largest E2M1 magnitude when s_b = s_raw.
  5. code_b = UE5M3 encode of s_raw (formats.ue5m3_encode); s_b = its value.
  6. If code_b is 0x00 (flushed to zero) or 0xFF (NaN): every element of the
     block keeps only its sign bit (magnitude index 0); 0xFF dequantizes to
     NaN.  Otherwise d = ts * s_b, r = 1 / d, v = x * r (one reciprocal per
     block, then one multiply per element).
  7. Magnitude index = round(|v|): nearest-even (formats.e2m1_round_nearest_even)
     or stochastic (formats.e2m1_round_stochastic) with the 16-bit values of
     philox.sr_bits.  The block scale itself is always rounded to nearest.
  8. Code = (sign bit of x) << 3 | index; the sign is copied even for zero
     magnitudes.  Byte j of an output row holds code 2j in its low nibble and
     code 2j+1 in its high nibble.  Scales are one byte per block, row-major.
"""

import numpy as np

from . import formats, philox

RNE = 0
SR = 1


def tensor_amax(x_bits):
    """max |x| over the whole bf16 tensor as float32 (a NaN propagates)."""
    x = formats.bf16_to_f32(x_bits)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def _quantize_rows(xo, ts, rounding, seed, offset, orientation, out_cols, row_ids):
    """Steps 3-8 for a set of output rows xo (fp32, shape (n, out_cols))."""
    n = xo.shape[0]
    nblk = out_cols // 16
    blocks = xo.reshape(n, nblk, 16)

    # 3. block amax
    amax_b = np.max(np.abs(blocks), axis=2)  # float32, NaN propagates

    # 4. raw block scale
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        K = np.float32(np.float32(6.0) * ts)  # +Inf for ts above fp32 max / 6
        s_raw = (amax_b / K).astype(np.float32)

    # 5. UE5M3 code and value
    code_b = formats.ue5m3_encode(s_raw)
    s_b = formats.ue5m3_decode(code_b).astype(np.float32)  # exact

    # 6. per-block reciprocal, per-element scaled value
    special = (code_b == 0x00) | (code_b == formats.UE5M3_NAN)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        d = (ts * np.where(special, np.float32(1.0), s_b)).astype(np.float32)
        r = (np.float32(1.0) / d).astype(np.float32)
        v = (blocks * r[:, :, None]).astype(np.float32)
    a = np.abs(v)

    # 7. rounding of the magnitude
    if rounding == RNE:
        idx = formats.e2m1_round_nearest_even(a)
    else:
        u16 = philox.sr_bits(seed, offset, orientation, None, out_cols, rows=row_ids)
        idx = formats.e2m1_round_stochastic(a, u16.reshape(n, nblk, 16))
    idx = np.where(special[:, :, None], 0, idx).astype(np.uint8)

    # 8. code with the sign of x, packed two per byte
    sign = np.signbit(blocks).astype(np.uint8)
    codes = ((sign << 3) | idx).reshape(n, out_cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, code_b.astype(np.uint8)


def quantize_blockscale(x_bits, ts, rounding=RNE, seed=0, offset=0, orientation=0,
                        rows=None, chunk=2048):
    """Quantize a bf16 tensor (uint16 bits, shape (R, C)) in one orientation.

    ts: the fp32 tensor scale.  orientation 0 -> codes (R, C/2), scales
    (R, C/16); orientation 1 -> codes (C, R/2), scales (C, R/16), i.e. the
    quantization of x^T.  rows: optional output-row indices to compute (a
    sample of a large output); the SR bits still use the true coordinates.
    Returns (codes uint8, scales uint8).
    """
    x = formats.bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    xo = x if orientation == 0 else x.T
    out_rows, out_cols = xo.shape
    if out_cols % 16 != 0:
        raise ValueError("the blocked axis must be a multiple of 16")
    ts = np.float32(ts)
    row_ids = np.arange(out_rows) if rows is None else np.asarray(rows, dtype=np.int64)
    codes = np.empty((len(row_ids), out_cols // 2), dtype=np.uint8)
    scales = np.empty((len(row_ids), out_cols // 16), dtype=np.uint8)
    for start in range(0, len(row_ids), chunk):
        ids = row_ids[start:start + chunk]
        sub = np.ascontiguousarray(xo[ids, :])
        c, s = _quantize_rows(sub, ts, rounding, seed, offset, orientation, out_cols, ids)
        codes[start:start + len(ids)] = c
        scales[start:start + len(ids)] = s
    return codes, scales


def unpack_codes(packed):
    """(n, C/2) packed bytes -> (n, C) codes 0..15 (low nibble first)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def dequantize_unscaled(packed, scales):
    """Exact q * s_b as float64, shape (n, C).  (q * s_b has at most 6
    significant bits and lies within [2^-18, 688128], so it is exact in fp32,
    bf16 and fp64 alike.)  Blocks with scale 0xFF give NaN."""
    q = formats.e2m1_decode(unpack_codes(packed))
    s = formats.ue5m3_decode(np.asarray(scales, dtype=np.uint8))
    n, c = q.shape
    return (q.reshape(n, c // 16, 16) * s[:, :, None]).reshape(n, c)


def dequantize(packed, scales, ts):
    """fp32 dequantization: float32(float32(q * s_b) * ts), one rounding."""
    qs = dequantize_unscaled(packed, scales).astype(np.float32)  # exact
    with np.errstate(invalid="ignore", over="ignore"):
        return (qs * np.float32(ts)).astype(np.float32)

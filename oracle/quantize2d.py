"""2-D (16 x 16) block-scaled E2M1/UE5M3 quantization (oracle side).

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this module.

[TIBQ] summary in the UE5M3 paper's related-papers list: with 1-D blocks a
tensor and its transpose get different scales, so the forward and the
backward GEMMs see differently quantized copies of the same values; 2-D
blocks make the scaling invariant under transposition, so one quantization
serves both orientations.  [UE5M3] abstract: UE5M3 scales, E2M1 payloads,
periodic fp32 tensor scale, stochastic rounding for backward gradients only.

Reading (the pages give the idea, not the arithmetic; the plainest version
consistent with the 1-D recipe in oracle/quantize.py):
  1. x = float32(bf16 bits << 16), shape (R, C); R and C are multiples of 16.
  2. Blocks: the aligned 16 x 16 tiles, tile (I, J) = rows 16I..16I+15,
     columns 16J..16J+15.
  3. amax_t = max |x| over the tile's 256 elements (a NaN propagates).
  4-6. As the 1-D recipe with amax_t in place of amax_b: K = 6 ts,
     s_raw = amax_t / K, code_t = UE5M3 encode, special codes 0x00 / 0xFF
     keep only the sign, otherwise r = 1 / (ts s_t) and v = x r.
  7. Rounding: nearest-even, or stochastic with the 16-bit value of element
     (i, j) taken from the row orientation's counter stream (orientation 0,
     output shape (R, C)), i.e. the bits the 1-D row-wise quantization of the
     same call would draw.  Each element is rounded once.
  8. The row-wise output packs the codes of each row (element 2j in the low
     nibble); the transposed output packs the same codes along the columns of
     x, so it is exactly the transpose of the row-wise codes.  Both outputs
     keep the 1-D layout of one scale byte per 16 elements of an output row:
     row_scales[i][J] = code_t(i // 16, J) and col_scales[j][I] =
     code_t(I, j // 16) -- the tile scale repeated over the tile's 16 rows
     (respectively columns) -- so the block-16 GEMMs consume both unchanged.
"""

import numpy as np

from . import formats, philox

RNE = 0
SR = 1


def tile_codes(x_bits, ts):
    """UE5M3 code of every 16 x 16 tile, shape (R/16, C/16) (steps 1-5)."""
    x = formats.bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    R, C = x.shape
    if R % 16 or C % 16:
        raise ValueError("both axes must be multiples of 16")
    tiles = np.abs(x).reshape(R // 16, 16, C // 16, 16)
    amax_t = np.max(np.max(tiles, axis=3), axis=1)  # float32, NaN propagates
    K = np.float32(np.float32(6.0) * np.float32(ts))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s_raw = (amax_t / K).astype(np.float32)
    return formats.ue5m3_encode(s_raw).astype(np.uint8)


def element_codes(x_bits, ts, rounding=RNE, seed=0, offset=0, row0=0):
    """E2M1 code (0..15) of every element, shape (R, C), and the tile codes.
    row0: x holds rows row0 .. row0 + R - 1 of a larger tensor with the same
    columns (a multiple of 16); the stochastic-rounding bits use the true row."""
    x = formats.bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    R, C = x.shape
    ts = np.float32(ts)
    code_t = tile_codes(x_bits, ts)
    # the tile code of every element
    code_e = np.repeat(np.repeat(code_t, 16, axis=0), 16, axis=1)
    s_e = formats.ue5m3_decode(code_e).astype(np.float32)  # exact
    special = (code_e == 0x00) | (code_e == formats.UE5M3_NAN)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        d = (ts * np.where(special, np.float32(1.0), s_e)).astype(np.float32)
        r = (np.float32(1.0) / d).astype(np.float32)
        v = (x * r).astype(np.float32)
    a = np.abs(v)
    if rounding == RNE:
        idx = formats.e2m1_round_nearest_even(a)
    else:
        u16 = philox.sr_bits(seed, offset, 0, None, C, rows=np.arange(row0, row0 + R))
        idx = formats.e2m1_round_stochastic(a, u16)
    idx = np.where(special, 0, idx).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8)
    return ((sign << 3) | idx).astype(np.uint8), code_t


def _pack(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def quantize_blockscale_2d(x_bits, ts, rounding=RNE, seed=0, offset=0, row0=0):
    """Quantize a bf16 tensor (uint16 bits, (R, C)) with 16 x 16 tile scales.

    Returns (row_codes (R, C/2), row_scales (R, C/16), col_codes (C, R/2),
    col_scales (C, R/16), tile_codes (R/16, C/16)), all uint8.  row0: as
    element_codes (a 16-aligned slice of rows of a larger tensor).
    """
    codes, code_t = element_codes(x_bits, ts, rounding, seed, offset, row0)
    row_codes = _pack(codes)
    col_codes = _pack(np.ascontiguousarray(codes.T))
    row_scales = np.repeat(code_t, 16, axis=0)
    col_scales = np.repeat(np.ascontiguousarray(code_t.T), 16, axis=0)
    return row_codes, row_scales, col_codes, col_scales, code_t

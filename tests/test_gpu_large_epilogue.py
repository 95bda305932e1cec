"""The quantizing GEMM epilogue past 2^35 outputs, where the stochastic
rounding call numbers (8 outputs per Philox call) pass 2^32 and need the
counter's second word.

Output 133120 x 262144 (532480 tiles; bf16 output 69.8 GB, each quantized
orientation 19.6 GB), K = 16, on exact-sum operands so the oracle has the
exact C.  Orientation 0's call numbers pass 2^32 at output row 131072,
orientation 1's (output rows = columns of C, 133120 long) inside column
258111.
Checks:
- sampled output rows and columns on both sides of those boundaries: the bf16
  values, and the codes and scales of both orientations, bit-exact with the
  oracle's rounding and stochastic quantization of the exact C;
- the whole output: every bf16 value finite (it starts as NaN, so a tile left
  unwritten fails), the amax equal to the largest stored magnitude, and the
  fused codes and scales equal to what the stand-alone quantizer (whose own
  past-2^35 parity is tested separately) writes for the stored output.
"Rethinking Shrinkage Bias in LLM FP4 Pretraining ... UFP4 Recipe",
abstract (stochastic rounding on dY, the three training GEMMs);
"format-aware fusion" article (quantization fused into the GEMM's output).
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, quantize
from oracle import gemm as ogemm

from devhelpers import dev_scalar, host

pytestmark = pytest.mark.gpu

M, N, K = 133120, 262144, 16
ROWS = [0, 1, 131071, 131072, 131073, M - 1]
COLS = [0, 7, 258111, 258112, 258113, N - 1]
EXACT_CODES = np.array([0, 1, 2, 8, 9, 10], dtype=np.uint8)  # 0, 0.5, 1 and their negatives
BAND = 8192


def _exact(rng, rows, ts):
    import torch

    nib = rng.choice(EXACT_CODES, size=(rows, K))
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0x78, 0x80, size=(rows, K // 16), dtype=np.uint8)
    q = lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), dev_scalar(ts))
    return q, codes, scales


def _exact_c(ac, asc, ta, bc, bsc, tb):
    ref, _ = ogemm.gemm_nt(ac, asc, ta, bc, bsc, tb)
    ref = ref + 0.0  # an exact zero is +0 (the accumulators start at +0)
    ref32 = ref.astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), ref), "operands do not give exact sums"
    return ref32


def test_boundaries():
    # row 131071 ends with call 2^32 - 1 and row 131072 starts with call 2^32;
    # column 258111 straddles 2^32 (its output row 2048 is the first past it)
    assert (131071 * N + N - 8) // 8 == 2**32 - 1 and (131072 * N) // 8 == 2**32
    assert 258111 * M + 2048 == 2**35 and 258112 * M > 2**35


def test_quantizing_epilogue_past_2_35_outputs(cuda_device):
    import torch

    rounding = lib.SR
    rng = np.random.default_rng(35)
    ta, tb = 0.5, 2.0 ** -9
    a, ac, asc = _exact(rng, M, ta)
    b, bc, bsc = _exact(rng, N, tb)
    R, Cc = np.array(ROWS, dtype=np.int64), np.array(COLS, dtype=np.int64)
    rows_bits = formats.f32_to_bf16_rne(_exact_c(ac[R], asc[R], ta, bc, bsc, tb))        # len(R) x N
    cols_bits = formats.f32_to_bf16_rne(_exact_c(ac, asc, ta, bc[Cc], bsc[Cc], tb))      # M x len(Cc)
    out_ts = np.float32(2.0 ** -14)
    seed, offset = 0x1234_5678_9ABC_DEF0, 41
    ts = dev_scalar(out_ts)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    qr, qc = lib.empty_quantized(M, N, ts), lib.empty_quantized(N, M, ts)
    lib.gemm_nt_bf16_quantized(a, b, y, ts, rounding, seed, offset, row=qr, col=qc, amax=amax)
    torch.cuda.synchronize()

    yi = y.view(torch.int16)
    assert np.array_equal(host(yi[R.tolist()]).view(np.uint16), rows_bits)
    assert np.array_equal(host(yi[:, Cc.tolist()]).view(np.uint16), cols_bits)
    for q, o, data, ids, n in ((qr, 0, rows_bits, R, N), (qc, 1, cols_bits.T, Cc, M)):
        c, s = quantize._quantize_rows(formats.bf16_to_f32(data), out_ts, rounding, seed, offset, o, n, ids)
        assert np.array_equal(host(q.scales[ids.tolist()]), s), f"scales, orientation {o}"
        assert np.array_equal(host(q.codes[ids.tolist()]), c), f"codes, orientation {o}"

    top = torch.zeros((), dtype=torch.float32, device="cuda")
    for r in range(0, M, BAND):
        band = y[r:r + BAND]
        assert bool(torch.isfinite(band).all()), f"non-finite output in rows {r}..{r + BAND}"
        top = torch.maximum(top, band.abs().max().float())
    assert host(amax)[0] == host(top.reshape(1))[0]

    sr, sc = lib.empty_quantized(M, N, ts), lib.empty_quantized(N, M, ts)
    lib.quantize_blockscale(y, ts, rounding, seed, offset, row=sr, col=sc)
    torch.cuda.synchronize()
    for fused, alone, n in ((qr, sr, M), (qc, sc, N)):
        for r in range(0, n, BAND):
            assert bool(torch.equal(fused.codes[r:r + BAND], alone.codes[r:r + BAND])), f"codes rows {r}.."
            assert bool(torch.equal(fused.scales[r:r + BAND], alone.scales[r:r + BAND])), f"scales rows {r}.."
    del a, b, y, yi, qr, qc, sr, sc
    torch.cuda.empty_cache()

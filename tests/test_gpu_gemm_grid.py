"""GPU parity of every GEMM instantiation on grids that take the tile order
the full-size launches take.

The GEMM kernels map workgroup ids to output tiles XCD by XCD (the first
8 * floor(tiles / 8) ids are regrouped so each XCD walks a contiguous range)
and then in groups of tile rows; grids of fewer than 8 tiles keep the plain
order.  These tests run grids of 32 to 90 tiles with several tile columns,
several tile-row groups, a ragged last group, ragged edge tiles and both the
aligned (K % 128 == 0) and the unaligned K paths, and compare the WHOLE
output with the oracle (outputs are prefilled with NaN, so a tile the order
skipped fails as well as a wrong one):
  - fp32 output (ue5m3fp4_gemm_nt): random codes over the full E2M1 and
    UE5M3 ranges, |C_gpu - C_ref| <= 1e-5 |tsA tsB| sum|a b| per element;
  - fp32, bf16 + amax and the quantizing epilogue on operands whose fp32
    partial sums are exact: bit-exact with the oracle's own rounding and
    quantization of C;
  - the native MXFP4 comparison GEMM, within the same tolerance.
"Rethinking Shrinkage Bias in LLM FP4 Pretraining ... UFP4 Recipe",
abstract: the three training GEMMs; "format-aware fusion" article: the fused
output and the MXFP4 route.
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, mxfp4, quantize
from oracle import gemm as ogemm

from devhelpers import assert_gemm_close, dev_scalar, host

pytestmark = pytest.mark.gpu

TILE = 256
# (M, N, K): tiles, tile-row groups of 4 -- 81 tiles (9 x 9, aligned K);
# 90 tiles (9 x 10, ragged M and N, unaligned K); 50 tiles (5 x 10, ragged
# K tail of 16); 32 tiles (16 x 2: eight groups of tall, narrow columns)
GRIDS = [(2304, 2304, 1024), (2080, 2320, 272), (1040, 2320, 400), (4096, 512, 128)]
EXACT_CODES = np.array([0, 1, 2, 8, 9, 10], dtype=np.uint8)  # 0, 0.5, 1 and their negatives


def tiles(M, N):
    return -(-M // TILE) * -(-N // TILE)


def _nan(m, n, dtype=None):
    import torch

    return torch.full((m, n), float("nan"), dtype=dtype or torch.float32, device="cuda")


def _device(codes, scales, ts):
    import torch

    return lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), dev_scalar(ts))


def _random(rng, rows, k, ts):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(0x01, 0xFF, size=(rows, k // 16), dtype=np.uint8)
    return _device(codes, scales, ts), codes, scales


def _exact(rng, rows, k, ts):
    nib = rng.choice(EXACT_CODES, size=(rows, k))
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0x78, 0x80, size=(rows, k // 16), dtype=np.uint8)
    return _device(codes, scales, ts), codes, scales


def _exact_c(ac, asc, ta, bc, bsc, tb):
    ref, _ = ogemm.gemm_nt(ac, asc, ta, bc, bsc, tb)
    ref = ref + 0.0  # an exact zero is +0 (the accumulators start at +0)
    ref32 = ref.astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), ref), "operands do not give exact sums"
    return ref32


def _bf16_bits(t):
    import torch

    return host(t.view(torch.int16)).view(np.uint16)


def test_grids_take_the_remapped_order():
    """The shapes above are the ones that exercise the XCD-remapped,
    grouped tile order (at least 8 tiles, several tile columns and groups)."""
    for M, N, _ in GRIDS:
        assert tiles(M, N) >= 32 and -(-N // TILE) >= 2
        assert -(-M // TILE) > 4  # more than one group of 4 tile rows


@pytest.mark.parametrize("M,N,K", GRIDS)
def test_fp32_full_range_whole_output(cuda_device, M, N, K):
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a, ac, asc = _random(rng, M, K, 0.75)
    b, bc, bsc = _random(rng, N, K, 1.5e-3)
    c = _nan(M, N)
    lib.gemm_nt(a, b, c)
    assert_gemm_close(host(c), ac, asc, 0.75, bc, bsc, 1.5e-3)


@pytest.mark.parametrize("M,N,K", GRIDS)
def test_fp32_and_bf16_exact_sums_whole_output(cuda_device, M, N, K):
    """Exact-sum operands: the fp32 output equals the exact C bit for bit;
    the bf16 output and its amax equal the oracle's rounding of it."""
    import torch

    rng = np.random.default_rng(M + 5 * N + 11 * K)
    a, ac, asc = _exact(rng, M, K, 0.5)
    b, bc, bsc = _exact(rng, N, K, 2.0 ** -6)
    ref32 = _exact_c(ac, asc, 0.5, bc, bsc, 2.0 ** -6)
    c = _nan(M, N)
    lib.gemm_nt(a, b, c)
    got = host(c)
    bad = np.argwhere(got.view(np.uint32) != ref32.view(np.uint32))
    assert bad.size == 0, f"fp32 output differs at {bad[:4].tolist()} (tiles {np.unique(bad // TILE, axis=0)[:4].tolist()})"
    y = _nan(M, N, torch.bfloat16)
    amax = dev_scalar(0.0)
    lib.gemm_nt_bf16(a, b, y, amax=amax)
    want = formats.f32_to_bf16_rne(ref32)
    bad = np.argwhere(_bf16_bits(y) != want)
    assert bad.size == 0, f"bf16 output differs at {bad[:4].tolist()}"
    assert host(amax)[0] == np.float32(np.max(np.abs(formats.bf16_to_f32(want))))


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
@pytest.mark.parametrize("M,N,K", [(2304, 2304, 1024), (2080, 2320, 272)])
def test_quantizing_epilogue_whole_output(cuda_device, rounding, M, N, K):
    """The quantizing epilogue on 81- and 90-tile grids: bf16 output, amax,
    and both quantized orientations of it bit-exact with the oracle's
    rounding and quantization of the exact C."""
    import torch

    rng = np.random.default_rng(M + N + K + rounding)
    a, ac, asc = _exact(rng, M, K, 0.5)
    b, bc, bsc = _exact(rng, N, K, 2.0 ** -8)
    ybits = formats.f32_to_bf16_rne(_exact_c(ac, asc, 0.5, bc, bsc, 2.0 ** -8))
    y32 = formats.bf16_to_f32(ybits)
    out_ts = np.float32(np.float32(np.max(np.abs(y32))) / np.float32(43008.0))
    ts = dev_scalar(out_ts)
    y = _nan(M, N, torch.bfloat16)
    amax = dev_scalar(0.0)
    qr, qc = lib.empty_quantized(M, N, ts), lib.empty_quantized(N, M, ts)
    qr.codes.fill_(0xAA), qr.scales.fill_(0xAA), qc.codes.fill_(0xAA), qc.scales.fill_(0xAA)
    lib.gemm_nt_bf16_quantized(a, b, y, ts, rounding, 77, 3, row=qr, col=qc, amax=amax)
    assert np.array_equal(_bf16_bits(y), ybits)
    assert host(amax)[0] == np.float32(np.max(np.abs(y32)))
    for q, o in ((qr, 0), (qc, 1)):
        oc, os_ = quantize.quantize_blockscale(ybits, out_ts, rounding, 77, 3, o)
        bad = np.argwhere(host(q.scales) != os_)
        assert bad.size == 0, f"orientation {o}: scale mismatch at {bad[:4].tolist()}"
        bad = np.argwhere(host(q.codes) != oc)
        assert bad.size == 0, f"orientation {o}: code mismatch at {bad[:4].tolist()}"


@pytest.mark.parametrize("M,N,K", [(2304, 2304, 1024), (2080, 2320, 288), (4096, 512, 256)])
def test_mxfp4_whole_output(cuda_device, M, N, K):
    import torch

    rng = np.random.default_rng(M + 3 * N + 7 * K)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    asc = rng.integers(100, 150, size=(M, K // 32), dtype=np.uint8)
    bsc = rng.integers(100, 150, size=(N, K // 32), dtype=np.uint8)
    out = _nan(M, N)
    lib.gemm_nt_mxfp4(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(0.5),
                      torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(3e-3), out)
    got = host(out).astype(np.float64)
    ref, bound = mxfp4.gemm_nt_mx(ac, asc, 0.5, bc, bsc, 3e-3)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    err = np.abs(got - ref)
    assert np.all(err <= 1e-5 * bound), f"worst excess {np.max(err - 1e-5 * bound):.3e}"


def _band_rows(n, seed, per_band=2):
    rng = np.random.default_rng(seed)
    pick = [0, n - 1]
    for b0 in range(0, n, TILE):
        size = min(TILE, n - b0)
        pick.extend(b0 + rng.choice(size, size=min(per_band, size), replace=False))
    return np.unique(np.asarray(pick, dtype=np.int64))


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
def test_quantizing_epilogue_ffn_shape_sampled(cuda_device, rounding):
    """The up projection's fprop shape, 8192 x 16384 x 4096 (2048 tiles), as
    the benchmark launches it, on exact-sum operands.  The oracle computes
    two full output rows and two full output columns in every 256-band (the
    exact C, rounded to bf16 by the oracle) and quantizes them: the bf16
    output, the row-wise codes and scales of those rows and the transposed
    ones of those columns are bit-exact with it.  Over the whole output the
    bf16 values are finite (every tile written), the fused codes and scales
    equal what the stand-alone quantizer writes for the stored output, and
    the amax is the max of the stored values."""
    import torch

    M, N, K = 8192, 16384, 4096
    rng = np.random.default_rng(4242 + rounding)
    a, ac, asc = _exact(rng, M, K, 0.5)
    b, bc, bsc = _exact(rng, N, K, 2.0 ** -9)
    R, Cc = _band_rows(M, 1), _band_rows(N, 2)
    # exact rows R and columns Cc of C, rounded to bf16 by the oracle
    rows32 = _exact_c(ac[R], asc[R], 0.5, bc, bsc, 2.0 ** -9)
    cols32 = _exact_c(ac, asc, 0.5, bc[Cc], bsc[Cc], 2.0 ** -9)
    ybits = np.zeros((M, N), dtype=np.uint16)  # only rows R and columns Cc are filled
    ybits[R, :] = formats.f32_to_bf16_rne(rows32)
    ybits[:, Cc] = formats.f32_to_bf16_rne(cols32)
    out_ts = np.float32(2.0 ** -14)
    ts = dev_scalar(out_ts)
    y = _nan(M, N, torch.bfloat16)
    amax = dev_scalar(0.0)
    qr, qc = lib.empty_quantized(M, N, ts), lib.empty_quantized(N, M, ts)
    lib.gemm_nt_bf16_quantized(a, b, y, ts, rounding, 91, 5, row=qr, col=qc, amax=amax)
    yb = _bf16_bits(y)
    assert np.array_equal(yb[R, :], ybits[R, :]) and np.array_equal(yb[:, Cc], ybits[:, Cc])
    for q, o, idx in ((qr, 0, R), (qc, 1, Cc)):
        oc, os_ = quantize.quantize_blockscale(ybits, out_ts, rounding, 91, 5, o, rows=idx)
        assert np.array_equal(host(q.scales)[idx], os_), f"orientation {o}: scales differ"
        assert np.array_equal(host(q.codes)[idx], oc), f"orientation {o}: codes differ"
    yf = y.float()
    assert bool(torch.isfinite(yf).all())
    assert host(amax)[0] == np.float32(host(yf.abs().max()))
    sr, sc = lib.empty_quantized(M, N, ts), lib.empty_quantized(N, M, ts)
    lib.quantize_blockscale(y, ts, rounding, 91, 5, row=sr, col=sc)
    for fused, alone in ((qr, sr), (qc, sc)):
        assert bool(torch.equal(fused.codes, alone.codes)) and bool(torch.equal(fused.scales, alone.scales))
    del a, b, y, yf, qr, qc, sr, sc
    torch.cuda.empty_cache()

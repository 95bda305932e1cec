"""GPU parity of the block-scaled GEMMs (HIP kernel through the C ABI).

C = tsA * tsB * A B^T with fp32 accumulation; several results are correct
(the accumulation order is free), so each element must satisfy
|C_gpu - C_oracle| <= 1e-5 * |tsA tsB| * sum_k |a_k b_k|.  Operands come from
the GPU quantizer, whose codes are bit-exact with the oracle (tested
separately); the oracle GEMM consumes the oracle's own codes of the same
bf16 inputs, which the GPU's must equal.  "Rethinking
Shrinkage Bias in LLM FP4 Pretraining ... UFP4 Recipe", abstract: the three
training GEMMs; "UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", abstract: UE5M3 block-16 operands.
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, quantize
from workloads import config, random_bf16, sr_seed, STALE_FACTORS

from devhelpers import (assert_gemm_close, assert_quant_equal, dev_bf16, dev_scalar,
                        fresh_ts, gpu_quantize, host, oracle_operand, sample_rows)

pytestmark = pytest.mark.gpu


def _empty(m, n):
    import torch

    return torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")


def _random_operand(rng, rows, k, lo=0x40, hi=0xB0, ts=1.0):
    import torch

    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, k // 16), dtype=np.uint8)
    q = lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                      dev_scalar(ts))
    return q, codes, scales


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 512), (300, 200, 4112),
                                   (1, 1, 16), (33, 130, 48), (129, 257, 144), (64, 64, 2048)])
def test_gemm_nt_random_codes_full(cuda_device, M, N, K):
    """Random code bytes and scales (including subnormal scales): whole
    output compared, multiple tiles, ragged M, N and K tails."""
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a, ac, asc = _random_operand(rng, M, K, 0x01, 0xFF, ts=0.75)
    b, bc, bsc = _random_operand(rng, N, K, 0x01, 0xFF, ts=1.5e-3)
    c = _empty(M, N)
    lib.gemm_nt(a, b, c)
    assert_gemm_close(host(c), ac, asc, 0.75, bc, bsc, 1.5e-3)


def test_gemm_k_zero_writes_zeros(cuda_device):
    import torch

    a = lib.Quantized(torch.zeros((4, 0), dtype=torch.uint8, device="cuda"),
                      torch.zeros((4, 0), dtype=torch.uint8, device="cuda"), dev_scalar(1.0))
    b = lib.Quantized(torch.zeros((3, 0), dtype=torch.uint8, device="cuda"),
                      torch.zeros((3, 0), dtype=torch.uint8, device="cuda"), dev_scalar(1.0))
    c = _empty(4, 3)
    lib.gemm_nt(a, b, c)
    assert np.all(host(c) == 0)


def test_gemm_nan_scale_row(cuda_device):
    rng = np.random.default_rng(5)
    a, ac, asc = _random_operand(rng, 64, 64)
    b, bc, bsc = _random_operand(rng, 48, 64)
    a.scales[7, 2] = 0xFF
    asc[7, 2] = 0xFF
    c = _empty(64, 48)
    lib.gemm_nt(a, b, c)
    got = host(c)
    assert np.all(np.isnan(got[7])) and np.isfinite(np.delete(got, 7, axis=0)).all()
    assert_gemm_close(got, ac, asc, 1.0, bc, bsc, 1.0)


def band_rows(n, seed, per_band=2, band=256):
    """per_band distinct random rows in every band of `band` rows (the GEMM's
    tile height and width), plus the first and the last row."""
    rng = np.random.default_rng(seed)
    pick = [0, n - 1]
    for b0 in range(0, n, band):
        size = min(band, n - b0)
        pick.extend(b0 + rng.choice(size, size=min(per_band, size), replace=False))
    return np.unique(np.asarray(pick, dtype=np.int64))


def _linear_layer(X, W, dY, seed, offset0=0, ts=None, rows_sample=None):
    """Quantize X, W (RNE) and dY (SR) in both orientations on the GPU and run
    fprop / dgrad / wgrad.  The oracle quantizes the same bf16 inputs itself
    -- at large sizes only the operand rows the sampled entries use, with
    their true coordinates -- the GPU codes must equal its codes, and the GEMM
    outputs must match the oracle GEMM on the oracle's operands.  At large
    sizes (rows_sample) the sampled operand rows are two per 256-row band of
    every operand, and the GEMM outputs are compared on every pair of them:
    at least four entries in every 256 x 256 output tile, whatever order the
    kernel walks its tiles in; the outputs start as NaN and must come out
    finite everywhere (every tile written)."""
    ts = ts or {}
    tsX = ts.get("X", fresh_ts(X))
    tsW = ts.get("W", fresh_ts(W))
    tsD = ts.get("dY", fresh_ts(dY))
    xr, xc = gpu_quantize(dev_bf16(X), tsX, lib.RNE)
    wr, wc = gpu_quantize(dev_bf16(W), tsW, lib.RNE)
    dr, dc = gpu_quantize(dev_bf16(dY), tsD, lib.SR, seed=seed, offset=offset0)
    tokens, in_f = X.shape
    out_f = W.shape[0]
    y, dx, dw = _empty(tokens, out_f), _empty(tokens, in_f), _empty(out_f, in_f)
    lib.gemm_fprop(xr, wr, y)
    lib.gemm_dgrad(dr, wc, dx)
    lib.gemm_wgrad(dc, xc, dw)
    if rows_sample:  # sampled tokens, output and input features: every tile band
        T = band_rows(tokens, 1)
        O = band_rows(out_f, 2)
        I = band_rows(in_f, 3)
    else:
        T, O, I = np.arange(tokens), np.arange(out_f), np.arange(in_f)
    # operand: GPU output, bf16 source, ts, rounding, seed, offset, orientation, output rows
    spec = {"Xr": (xr, X, tsX, lib.RNE, 0, 0, 0, T), "Xc": (xc, X, tsX, lib.RNE, 0, 0, 1, I),
            "Wr": (wr, W, tsW, lib.RNE, 0, 0, 0, O), "Wc": (wc, W, tsW, lib.RNE, 0, 0, 1, I),
            "Dr": (dr, dY, tsD, lib.SR, seed, offset0, 0, T), "Dc": (dc, dY, tsD, lib.SR, seed, offset0, 1, O)}
    ops = {}
    for name, (q, bits, t, rnd, sd, off, o, idx) in spec.items():
        ops[name] = oracle_operand(bits, t, rnd, sd, off, o, q_gpu=q, rows=idx if rows_sample else None) + (idx,)
    worst = 0.0
    for c, ka, kb, ta, tb in ((y, "Xr", "Wr", tsX, tsW), (dx, "Dr", "Wc", tsD, tsW), (dw, "Dc", "Xc", tsD, tsX)):
        ac, asc, ra = ops[ka]
        bc, bsc, rb = ops[kb]
        got = host(c)
        if rows_sample:
            assert np.isfinite(got).all(), f"{ka}x{kb}: output entries left unwritten or not finite"
            tiles_hit = {(i // 256, j // 256) for i in ra for j in rb}
            assert len(tiles_hit) == (-(-got.shape[0] // 256)) * (-(-got.shape[1] // 256))
            e = assert_gemm_close(got[np.ix_(ra, rb)], ac, asc, ta, bc, bsc, tb)
        else:
            e = assert_gemm_close(got, ac, asc, ta, bc, bsc, tb)
        worst = max(worst, e)
    return dict(X=(xr, xc, tsX), W=(wr, wc, tsW), dY=(dr, dc, tsD), worst=worst)


def test_config1_roundtrip_and_fprop(cuda_device):
    """256 x 256 X and W ~ N(0,1), seed 0, fresh tensor scales, RNE: codes,
    scales and dequantization bit-exact; fprop within tolerance."""
    import torch

    data = config(1)
    X, W = data["X"], data["W"]
    tsX, tsW = fresh_ts(X), fresh_ts(W)
    xr, _ = gpu_quantize(dev_bf16(X), tsX, lib.RNE, col=False)
    wr, _ = gpu_quantize(dev_bf16(W), tsW, lib.RNE, col=False)
    ox = oracle_operand(X, tsX, lib.RNE, 0, 0, 0, q_gpu=xr)
    ow = oracle_operand(W, tsW, lib.RNE, 0, 0, 0, q_gpu=wr)
    for q, (oc, os_), ts in ((xr, ox, tsX), (wr, ow, tsW)):
        out = torch.empty((256, 256), dtype=torch.float32, device="cuda")
        lib.dequantize(q, out)
        ref = quantize.dequantize(oc, os_, ts)
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
    y = _empty(256, 256)
    lib.gemm_fprop(xr, wr, y)
    assert_gemm_close(host(y), ox[0], ox[1], tsX, ow[0], ow[1], tsW)


def test_small_linear_layer_full(cuda_device):
    X = random_bf16((272, 400), seed=1)
    W = random_bf16((176, 400), seed=2, kind="heavy")
    dY = random_bf16((272, 176), seed=3, kind="gradient")
    r = _linear_layer(X, W, dY, seed=17)
    for name, bits in (("X", X), ("W", W), ("dY", dY)):
        qr, qc, ts = r[name]
        rnd = lib.SR if name == "dY" else lib.RNE
        assert_quant_equal(qr, bits, ts, rnd, 17 if rnd else 0, 0, 0)
        assert_quant_equal(qc, bits, ts, rnd, 17 if rnd else 0, 0, 1)


def test_config3_attention_projection(cuda_device):
    """tokens 8192, in 4096, out 4096: fprop / dgrad / wgrad, SR on dY only."""
    d = config(3)
    r = _linear_layer(d["X"], d["W"], d["dY"], seed=sr_seed(3), rows_sample=400)
    for name in ("X", "W", "dY"):
        qr, qc, ts = r[name]
        bits = d[name]
        rnd = lib.SR if name == "dY" else lib.RNE
        seed = sr_seed(3) if rnd else 0
        assert_quant_equal(qr, bits, ts, rnd, seed, 0, 0, rows=sample_rows(bits.shape[0], 24, 5))
        assert_quant_equal(qc, bits, ts, rnd, seed, 0, 1, rows=sample_rows(bits.shape[1], 24, 6))


def test_config4_ffn_pair(cuda_device):
    """FFN up (4096 -> 16384) and down (16384 -> 4096) layers at 8192 tokens:
    six GEMMs, each 8192 x 4096 x 16384 in some order, in the launch
    configuration the benchmark times; at least four sampled entries in every
    one of their 512-2048 output tiles."""
    d = config(4)
    _linear_layer(d["X"], d["W_up"], d["dY_up"], seed=sr_seed(4), offset0=0, rows_sample=300)
    _linear_layer(d["H"], d["W_down"], d["dY_down"], seed=sr_seed(4), offset0=1, rows_sample=300)


@pytest.mark.parametrize("factor", STALE_FACTORS)
def test_config5_gemms_with_stale_scales(cuda_device, factor):
    d = config(5)
    ts = {}
    for name in ("X", "W", "dY"):
        a = quantize.tensor_amax(d[name]) * np.float32(factor)
        ts[name] = np.float32(a / np.float32(43008.0))
    _linear_layer(d["X"], d["W"], d["dY"], seed=sr_seed(5), ts=ts, rows_sample=400)


def test_dequant_exhaustive_through_gemm(cuda_device):
    """Every (E2M1 code, UE5M3 scale) pair, exactly: row i of A holds pair i at
    k = 0 (zeros elsewhere), B has a single 1.0 (code 2, scale 0x78) at k = 0,
    so C[i][0] = q * s must come out exact.  Repeated at every position of a
    128-element K chunk to cover every lane and nibble of the fragment layout."""
    import torch

    codes_q = np.arange(16)
    codes_s = np.arange(256)
    pairs = np.array([(c, s) for s in codes_s for c in codes_q])  # 4096 pairs
    M, K = len(pairs), 128
    for pos in (0, 1, 7, 8, 15, 16, 33, 64, 100, 127):
        ac = np.zeros((M, K // 2), np.uint8)
        asc = np.full((M, K // 16), 0x78, np.uint8)
        byte = pos // 2
        ac[:, byte] = (pairs[:, 0] << (4 * (pos % 2))).astype(np.uint8)
        asc[:, pos // 16] = pairs[:, 1]
        bc = np.zeros((16, K // 2), np.uint8)
        bsc = np.full((16, K // 16), 0x78, np.uint8)
        bc[0, byte] = 2 << (4 * (pos % 2))  # 1.0
        a = lib.Quantized(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(1.0))
        b = lib.Quantized(torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(1.0))
        c = _empty(M, 16)
        lib.gemm_nt(a, b, c)
        got = host(c)[:, 0].astype(np.float64)
        ref = formats.e2m1_decode(pairs[:, 0]) * formats.ue5m3_decode(pairs[:, 1])
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), pos
        assert np.array_equal(got[~nan], ref[~nan]), (pos, np.argwhere(got[~nan] != ref[~nan])[:4])
        rest = host(c)[:, 1:]  # B rows of zeros: 0, or NaN where A's block scale is NaN
        assert np.all(rest[~nan] == 0) and np.all(np.isnan(rest[nan]))


def _fp32_down(x):
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f)


def _fp32_up(x):
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f)


def _bf16_rne(f32):
    """fp32 -> bf16 value (round to nearest even) by torch's CPU cast."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(f32)).to(torch.bfloat16).to(torch.float32).numpy()


@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (300, 200, 4112), (33, 130, 48), (1, 1, 16)])
def test_gemm_nt_bf16_with_amax(cuda_device, M, N, K):
    """Fused epilogue: bf16 output and its amax.  Each bf16 value must be the
    round-to-nearest-even image of some fp32 within the GEMM tolerance of the
    oracle (rounding is monotone, so it lies between the images of the ends of
    that interval); the amax must be the max |.| of the values stored."""
    import torch

    rng = np.random.default_rng(M + 5 * N + 11 * K)
    a, ac, asc = _random_operand(rng, M, K, 0x40, 0xB0, ts=0.5)
    b, bc, bsc = _random_operand(rng, N, K, 0x40, 0xB0, ts=2.0e-3)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    lib.gemm_nt_bf16(a, b, out, amax=amax)
    got = out.to(torch.float32).cpu().numpy().astype(np.float64)
    from oracle import gemm as ogemm

    ref, bound = ogemm.gemm_nt(ac, asc, 0.5, bc, bsc, 2.0e-3)
    tol = 1e-5 * bound
    lo = _bf16_rne(_fp32_down(ref - tol)).astype(np.float64)
    hi = _bf16_rne(_fp32_up(ref + tol)).astype(np.float64)
    bad = np.argwhere((got < lo) | (got > hi))
    assert bad.size == 0, f"bf16 output outside the rounded tolerance band at {bad[:3].tolist()}"
    assert host(amax)[0] == np.float32(np.max(np.abs(got)))
    # a larger running amax is left alone
    big = dev_scalar(1e30)
    lib.gemm_nt_bf16(a, b, out, amax=big)
    assert host(big)[0] == np.float32(1e30)


def test_gemm_nt_bf16_nan_block(cuda_device):
    """A NaN block scale (0xFF) poisons its output row in bf16 and the amax."""
    import torch

    rng = np.random.default_rng(3)
    a, ac, asc = _random_operand(rng, 40, 64, 0x40, 0xB0)
    b, bc, bsc = _random_operand(rng, 24, 64, 0x40, 0xB0)
    asc[7, 2] = 0xFF
    a = lib.Quantized(a.codes, torch.from_numpy(asc).cuda(), a.ts)
    out = torch.empty((40, 24), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    lib.gemm_nt_bf16(a, b, out, amax=amax)
    got = out.to(torch.float32).cpu().numpy()
    assert np.all(np.isnan(got[7])) and not np.any(np.isnan(np.delete(got, 7, axis=0)))
    assert np.isnan(host(amax)[0])


@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (300, 200, 4112), (33, 130, 48), (1, 1, 16), (520, 272, 1024)])
def test_gemm_exact_sums_bit_exact(cuda_device, M, N, K):
    """Operands on which every fp32 partial sum is exact -- payload
    magnitudes 0, 0.5 and 1, scales in [1, 1.875], power-of-two tensor
    scales: each product is a multiple of 2^-8 below 3.6, so for K <= 4112
    every partial sum is a multiple of 2^-8 below 2^14 (22 significant bits)
    whatever the order.  The fp32 output must then equal the oracle's exact
    result bit for bit, and the bf16 output and its amax the oracle's
    round-to-nearest-even image of it."""
    import torch

    rng = np.random.default_rng(M + 13 * N + K)
    vals = np.array([0, 1, 2, 8, 9, 10], dtype=np.uint8)
    ops = []
    for rows, ts in ((M, 0.5), (N, 2.0 ** -6)):
        nib = rng.choice(vals, size=(rows, K))
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales = rng.integers(0x78, 0x80, size=(rows, K // 16), dtype=np.uint8)
        q = lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), dev_scalar(ts))
        ops.append((q, codes, scales, ts))
    (a, ac, asc, ta), (b, bc, bsc, tb) = ops
    from oracle import gemm as ogemm

    ref, _ = ogemm.gemm_nt(ac, asc, ta, bc, bsc, tb)
    ref = ref + 0.0  # an exact zero is +0 (the accumulators start at +0)
    ref32 = ref.astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), ref)  # the construction is exact
    c = _empty(M, N)
    lib.gemm_nt(a, b, c)
    assert np.array_equal(host(c).view(np.uint32), ref32.view(np.uint32))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    lib.gemm_nt_bf16(a, b, out, amax=amax)
    want = formats.f32_to_bf16_rne(ref32)
    assert np.array_equal(host(out.view(torch.int16)).view(np.uint16), want)
    assert host(amax)[0] == np.float32(np.max(np.abs(formats.bf16_to_f32(want))))

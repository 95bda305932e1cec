"""GPU parity of the block-scaled GEMMs (HIP kernel through the C ABI).

C = tsA * tsB * A B^T with fp32 accumulation; several results are correct
(the accumulation order is free), so each element must satisfy
|C_gpu - C_oracle| <= 1e-5 * |tsA tsB| * sum_k |a_k b_k|.  Operands come from
the GPU quantizer, whose codes are bit-exact with the oracle (tested
separately); the oracle GEMM consumes the same code bytes.  "Rethinking
Shrinkage Bias in LLM FP4 Pretraining ... UFP4 Recipe", abstract: the three
training GEMMs; "UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", abstract: UE5M3 block-16 operands.
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, quantize
from workloads import config, random_bf16, sr_seed, STALE_FACTORS

from devhelpers import (assert_gemm_close, assert_quant_equal, dev_bf16, dev_scalar, fresh_ts,
                        gpu_quantize, host, sample_rows)

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


def _linear_layer(X, W, dY, seed, offset0=0, ts=None, rows_sample=None):
    """Quantize X, W (RNE) and dY (SR) in both orientations on the GPU, check
    the codes against the oracle, run fprop / dgrad / wgrad and check them."""
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
    worst = 0.0
    for c, (qa, ta), (qb, tb) in ((y, (xr, tsX), (wr, tsW)), (dx, (dr, tsD), (wc, tsW)),
                                  (dw, (dc, tsD), (xc, tsX))):
        got = host(c)
        m, n = got.shape
        if rows_sample:
            rng = np.random.default_rng(m + n)
            rr = rng.integers(0, m, rows_sample)
            cc = rng.integers(0, n, rows_sample)
            rr[:2], cc[:2] = [0, m - 1], [0, n - 1]
            e = assert_gemm_close(got, host(qa.codes), host(qa.scales), ta, host(qb.codes),
                                  host(qb.scales), tb, rr, cc)
        else:
            e = assert_gemm_close(got, host(qa.codes), host(qa.scales), ta, host(qb.codes),
                                  host(qb.scales), tb)
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
    assert_quant_equal(xr, X, tsX, lib.RNE, 0, 0, 0)
    assert_quant_equal(wr, W, tsW, lib.RNE, 0, 0, 0)
    for q, ts in ((xr, tsX), (wr, tsW)):
        out = torch.empty((256, 256), dtype=torch.float32, device="cuda")
        lib.dequantize(q, out)
        ref = quantize.dequantize(host(q.codes), host(q.scales), ts)
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
    y = _empty(256, 256)
    lib.gemm_fprop(xr, wr, y)
    assert_gemm_close(host(y), host(xr.codes), host(xr.scales), tsX, host(wr.codes),
                      host(wr.scales), tsW)


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
    r = _linear_layer(d["X"], d["W"], d["dY"], seed=sr_seed(3), rows_sample=1500)
    for name in ("X", "W", "dY"):
        qr, qc, ts = r[name]
        bits = d[name]
        rnd = lib.SR if name == "dY" else lib.RNE
        seed = sr_seed(3) if rnd else 0
        assert_quant_equal(qr, bits, ts, rnd, seed, 0, 0, rows=sample_rows(bits.shape[0], 24, 5))
        assert_quant_equal(qc, bits, ts, rnd, seed, 0, 1, rows=sample_rows(bits.shape[1], 24, 6))


def test_config4_ffn_pair(cuda_device):
    """FFN up (4096 -> 16384) and down (16384 -> 4096) layers at 8192 tokens:
    six GEMMs, each 8192 x 4096 x 16384 in some order, on sampled entries."""
    d = config(4)
    _linear_layer(d["X"], d["W_up"], d["dY_up"], seed=sr_seed(4), offset0=0, rows_sample=600)
    _linear_layer(d["H"], d["W_down"], d["dY_down"], seed=sr_seed(4), offset0=1, rows_sample=600)


@pytest.mark.parametrize("factor", STALE_FACTORS)
def test_config5_gemms_with_stale_scales(cuda_device, factor):
    d = config(5)
    ts = {}
    for name in ("X", "W", "dY"):
        a = quantize.tensor_amax(d[name]) * np.float32(factor)
        ts[name] = np.float32(a / np.float32(43008.0))
    _linear_layer(d["X"], d["W"], d["dY"], seed=sr_seed(5), ts=ts, rows_sample=1500)


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

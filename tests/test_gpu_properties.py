"""Whole-output checks at the benchmark's full sizes, from properties that hold
for every input and every size.  At these sizes the oracle comparisons are
sampled (tests/test_gpu_gemm.py, tests/test_gpu_quantize.py); here every
output element of full-size launches in the launch configuration the
benchmark times is checked against another launch:

- sign symmetry: the block scale depends on |x| and each payload rounds |v|
  and copies x's sign, so quantizing -x gives the same scales and codes with
  every sign bit flipped -- for stochastic rounding too (the random bits
  depend on coordinates only);
- power-of-two equivariance: scaling x and the tensor scale by 2^k scales
  amax, K = 6 ts and ts * s_b by 2^k and r by 2^-k, all exactly, so the
  scales and codes are unchanged (both roundings);
- transpose consistency (round to nearest, whose codes do not depend on
  coordinates): the transposed output of x is the row-wise output of x^T;
- GEMM: doubling tsA doubles C exactly (the epilogue is (acc * 256 tsA) *
  tsB); reversing the order of A's (or B's) 32-row groups, which keeps every
  row's place inside its 32 x 32 MFMA block but moves it to other tiles and
  XCDs, permutes C's rows (columns) the same way, bit for bit -- for the fp32
  output, the bf16 + amax output, the quantizing epilogue (RNE, both
  orientations) and the native MXFP4 GEMM;
- 2-D (16 x 16 tile) scales: each element is rounded once, so the transposed
  codes are the row-wise codes transposed and both scale outputs repeat the
  tile scale (both roundings).

Inputs: config 4's X (8192 x 4096), W_up (16384 x 4096) and dY_up
(8192 x 16384), the tensor scale refreshed from each tensor's amax.
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from devhelpers import dev_bf16, dev_scalar, fresh_ts
from workloads import config, sr_seed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c4(cuda_device):
    import torch

    d = config(4)
    data = {k: d[k] for k in ("X", "W_up", "dY_up")}
    del d
    yield data
    torch.cuda.empty_cache()


def quant(x_dev, ts, rounding, seed=0, offset=0, col=True):
    rows, cols = x_dev.shape
    ts_dev = dev_scalar(ts)
    qr = lib.empty_quantized(rows, cols, ts_dev)
    qc = lib.empty_quantized(cols, rows, ts_dev) if col else None
    lib.quantize_blockscale(x_dev, ts_dev, rounding, seed, offset, row=qr, col=qc)
    return qr, qc


def same(a, b):
    import torch

    torch.cuda.synchronize()
    return torch.equal(a, b)


@pytest.mark.parametrize("name,rounding", [("dY_up", lib.SR), ("dY_up", lib.RNE), ("X", lib.RNE)])
def test_sign_symmetry_whole_output(c4, name, rounding):
    import torch

    bits = c4[name]
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    neg = x ^ torch.tensor(-32768, dtype=torch.int16, device="cuda")  # flip every bf16 sign bit
    seed, offset = sr_seed(4), 11
    pr, pc = quant(x, ts, rounding, seed, offset)
    nr, nc = quant(neg, ts, rounding, seed, offset)
    del x, neg
    flip = torch.tensor(0x88, dtype=torch.uint8, device="cuda")
    for p, n, what in ((pr, nr, "row-wise"), (pc, nc, "transposed")):
        assert same(p.scales, n.scales), f"{what} scales differ"
        assert same(p.codes ^ flip, n.codes), f"{what} codes are not sign-flipped"


@pytest.mark.parametrize("k", [5, -7])
@pytest.mark.parametrize("name,rounding", [("dY_up", lib.SR), ("X", lib.RNE)])
def test_power_of_two_equivariance_whole_output(c4, name, rounding, k):
    import torch

    bits = c4[name]
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    xs = (x.view(torch.bfloat16) * (2.0 ** k)).view(torch.int16)  # exact: no bf16 overflow or underflow here
    assert torch.equal((xs.view(torch.bfloat16) * (2.0 ** -k)).view(torch.int16), x)
    seed, offset = sr_seed(4), 3
    ar, ac = quant(x, ts, rounding, seed, offset)
    br, bc = quant(xs, np.float32(ts * np.float32(2.0 ** k)), rounding, seed, offset)
    del x, xs
    for a, b, what in ((ar, br, "row-wise"), (ac, bc, "transposed")):
        assert same(a.scales, b.scales), f"{what} scales differ"
        assert same(a.codes, b.codes), f"{what} codes differ"


@pytest.mark.parametrize("name", ["W_up", "dY_up"])
def test_transpose_consistency_whole_output(c4, name):
    bits = c4[name]
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    xt = x.t().contiguous()
    _, qc = quant(x, ts, lib.RNE)
    tr, _ = quant(xt, ts, lib.RNE, col=False)
    del x, xt
    assert same(qc.scales, tr.scales)
    assert same(qc.codes, tr.codes)


@pytest.fixture(scope="module")
def up_operands(c4):
    """X and W_up quantized row-wise (the up projection's fprop operands)."""
    out = []
    for name in ("X", "W_up"):
        q, _ = quant(dev_bf16(c4[name]), fresh_ts(c4[name]), lib.RNE, col=False)
        out.append(q)
    return out


def test_gemm_tensor_scale_linearity_whole_output(up_operands):
    import torch

    a, b = up_operands
    M, N = a.rows, b.rows
    c1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    c2 = torch.empty_like(c1)
    lib.gemm_nt(a, b, c1)
    a2 = lib.Quantized(a.codes, a.scales, a.ts * 2.0)
    lib.gemm_nt(a2, b, c2)
    assert same(c2, c1 * 2.0)
    assert bool(torch.isfinite(c1).all())


def _reverse_groups(n):
    import torch

    return torch.arange(n, device="cuda").view(n // 32, 32).flip(0).reshape(-1)


@pytest.mark.parametrize("operand", ["A", "B"])
def test_gemm_tile_permutation_whole_output(up_operands, operand):
    import torch

    a, b = up_operands
    M, N = a.rows, b.rows
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    cp = torch.empty_like(c)
    lib.gemm_nt(a, b, c)
    if operand == "A":
        idx = _reverse_groups(M)
        ap = lib.Quantized(a.codes[idx].contiguous(), a.scales[idx].contiguous(), a.ts)
        lib.gemm_nt(ap, b, cp)
        assert same(cp, c[idx])
    else:
        idx = _reverse_groups(N)
        bp = lib.Quantized(b.codes[idx].contiguous(), b.scales[idx].contiguous(), b.ts)
        lib.gemm_nt(a, bp, cp)
        assert same(cp, c[:, idx])


def _unpack(codes):
    """[R][C/2] packed nibbles (element 2j low) -> [R][C] uint8 codes."""
    import torch

    return torch.stack((codes & 0x0F, codes >> 4), dim=2).reshape(codes.shape[0], -1)


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
def test_2d_transposed_output_is_the_transpose_whole_output(c4, rounding):
    """2-D (16 x 16 tile) scales round each element once: the transposed
    codes are the row-wise codes transposed, and both scale outputs repeat
    the tile scale (dY_up, 8192 x 16384)."""
    import torch

    bits = c4["dY_up"]
    R, C = bits.shape
    ts = dev_scalar(fresh_ts(bits))
    x = dev_bf16(bits)
    qr, qc = lib.empty_quantized(R, C, ts), lib.empty_quantized(C, R, ts)
    lib.quantize_blockscale_2d(x, ts, rounding, sr_seed(4), 21, row=qr, col=qc)
    del x
    assert same(_unpack(qc.codes), _unpack(qr.codes).t().contiguous())
    tiles = qr.scales[::16]                                           # [R/16][C/16]
    assert same(qr.scales, tiles.repeat_interleave(16, dim=0))
    assert same(qc.scales, tiles.t().contiguous().repeat_interleave(16, dim=0))


@pytest.mark.parametrize("operand", ["A", "B"])
def test_gemm_bf16_tile_permutation_whole_output(up_operands, operand):
    """The bf16 + amax epilogue at the up projection's fprop shape (2048
    tiles): reversing A's (B's) 32-row groups permutes the output's rows
    (columns) bit for bit and keeps the amax."""
    import torch

    a, b = up_operands
    M, N = a.rows, b.rows
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yp = torch.empty_like(y)
    am, amp = dev_scalar(0.0), dev_scalar(0.0)
    lib.gemm_nt_bf16(a, b, y, amax=am)
    if operand == "A":
        idx = _reverse_groups(M)
        lib.gemm_nt_bf16(lib.Quantized(a.codes[idx].contiguous(), a.scales[idx].contiguous(), a.ts), b, yp, amax=amp)
        assert same(yp.view(torch.int16), y.view(torch.int16)[idx])
    else:
        idx = _reverse_groups(N)
        lib.gemm_nt_bf16(a, lib.Quantized(b.codes[idx].contiguous(), b.scales[idx].contiguous(), b.ts), yp, amax=amp)
        assert same(yp.view(torch.int16), y.view(torch.int16)[:, idx])
    assert same(am, amp)


def test_quantizing_epilogue_tile_permutation_whole_output(up_operands):
    """The quantizing epilogue (RNE, both orientations) at the same shape:
    reversing A's 32-row groups permutes the bf16 output's rows, the
    row-wise codes' and scales' rows, and in the transposed output each
    row's 16-byte code groups and 2-byte scale groups (a 32-row group is 16
    code bytes and 2 scale bytes there); the amax is kept."""
    import torch

    a, b = up_operands
    M, N = a.rows, b.rows
    ts = dev_scalar(2.0 ** -10)
    idx = _reverse_groups(M)
    ap = lib.Quantized(a.codes[idx].contiguous(), a.scales[idx].contiguous(), a.ts)
    outs = []
    for opa in (a, ap):
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        qr, qc = lib.empty_quantized(M, N, ts), lib.empty_quantized(N, M, ts)
        am = dev_scalar(0.0)
        lib.gemm_nt_bf16_quantized(opa, b, y, ts, lib.RNE, row=qr, col=qc, amax=am)
        outs.append((y, qr, qc, am))
    (y, qr, qc, am), (yp, qrp, qcp, amp) = outs
    g = M // 32
    assert same(yp.view(torch.int16), y.view(torch.int16)[idx])
    assert same(qrp.codes, qr.codes[idx]) and same(qrp.scales, qr.scales[idx])
    assert same(qcp.codes.view(N, g, 16), qc.codes.view(N, g, 16).flip(1))
    assert same(qcp.scales.view(N, g, 2), qc.scales.view(N, g, 2).flip(1))
    assert same(am, amp)


def test_mxfp4_tile_permutation_whole_output(cuda_device):
    """The native MXFP4 GEMM at the benchmark's shape (8192 x 4096 x 16384,
    512 tiles): reversing A's 32-row groups permutes C's rows bit for bit."""
    import torch

    M, N, K = 8192, 4096, 16384
    g = torch.Generator(device="cuda").manual_seed(29)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    bc = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    asc = torch.randint(110, 140, (M, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    bsc = torch.randint(110, 140, (N, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    one = dev_scalar(1.0)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    cp = torch.empty_like(c)
    lib.gemm_nt_mxfp4(ac, asc, one, bc, bsc, one, c)
    idx = _reverse_groups(M)
    lib.gemm_nt_mxfp4(ac[idx].contiguous(), asc[idx].contiguous(), one, bc, bsc, one, cp)
    assert same(cp, c[idx])
    assert bool(torch.isfinite(c).all())

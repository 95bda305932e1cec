"""Maximum-size edge cases: tensors past 2^31 elements and GEMM outputs past
2^31 entries, so every byte offset needs 64 bits.  The input is a seeded
block from the input generator (4093 x 16384: a row period that is not a
power of two, so an offset that wrapped would read different data) tiled on
the device to 133120 rows; sampled rows / entries are compared with the
oracle on the generator's block (round to nearest: the codes do not depend
on coordinates, so a sampled row can be quantized on its own).

Sizes: x is 133120 x 16384 bf16 (2.18e9 elements, 4.4 GB; outputs 1.2 GB per
orientation); C is 65536 x 36864 fp32 (2.4e9 entries, 9.7 GB).  Past 2^35
elements (below) the stochastic-rounding counters take their 64-bit form:
there x is 133120 x 262144 (69.8 GB), checked through the 1-D and the 2-D
quantizer."""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import quantize, quantize2d
from workloads import random_bf16

from devhelpers import dev_bf16, dev_scalar, host

pytestmark = pytest.mark.gpu

R, C = 133120, 16384
PERIOD = 4093
ROWS = np.array([0, 1, 8191, 65535, 65536, 131071, 131072, R - 16, R - 1])
COLS = [0, 7, 4096, C - 1]


@pytest.fixture(scope="module")
def big_x(cuda_device):
    import torch

    block = random_bf16((PERIOD, C), seed=20260)
    blk = dev_bf16(block)
    x = blk.repeat(-(-R // PERIOD), 1)[:R].contiguous()
    del blk
    assert x.numel() > 2**31
    yield block, x
    del x
    torch.cuda.empty_cache()


def test_quantize_past_2_31_elements(big_x):
    import torch

    block, x = big_x
    amax_ref = quantize.tensor_amax(block)
    ts_val = np.float32(np.float32(amax_ref) / np.float32(43008.0))
    ts = dev_scalar(ts_val)
    amax = dev_scalar(0.0)
    qr = lib.empty_quantized(R, C, ts)
    qc = lib.empty_quantized(C, R, ts)
    lib.quantize_blockscale(x, ts, lib.RNE, row=qr, col=qc, amax=amax)
    torch.cuda.synchronize()
    assert host(amax)[0] == amax_ref
    c, s = quantize.quantize_blockscale(block[ROWS % PERIOD], ts_val, quantize.RNE)
    assert np.array_equal(host(qr.codes[ROWS.tolist()]), c) and np.array_equal(host(qr.scales[ROWS.tolist()]), s)
    cols = np.tile(block[:, COLS], (-(-R // PERIOD), 1))[:R]  # R x k: output rows of the transposed orientation
    c, s = quantize.quantize_blockscale(cols, ts_val, quantize.RNE, orientation=1)
    assert np.array_equal(host(qc.codes[COLS]), c) and np.array_equal(host(qc.scales[COLS]), s)
    del qr, qc


def test_quantize_2d_past_2_31_elements(big_x):
    import torch

    block, x = big_x
    ts_val = np.float32(np.float32(quantize.tensor_amax(block)) / np.float32(43008.0))
    ts = dev_scalar(ts_val)
    qr = lib.empty_quantized(R, C, ts)
    qc = lib.empty_quantized(C, R, ts)
    lib.quantize_blockscale_2d(x, ts, lib.RNE, row=qr, col=qc)
    torch.cuda.synchronize()
    for g in (0, 4096, 8192, R // 16 - 1):  # 16-row groups (8192: rows 131072.., past 2^31 elements)
        xs = block[(16 * g + np.arange(16)) % PERIOD]
        rc, rs, cc, cs, _ = quantize2d.quantize_blockscale_2d(xs, ts_val, quantize.RNE)
        assert np.array_equal(host(qr.codes[16 * g:16 * g + 16]), rc)
        assert np.array_equal(host(qr.scales[16 * g:16 * g + 16]), rs)
        assert np.array_equal(host(qc.codes[:, 8 * g:8 * g + 8]), cc)
        assert np.array_equal(host(qc.scales[:, g:g + 1]), cs)
    del qr, qc


def test_current_scaling_past_2_31_elements(big_x):
    """Current-tensor scaling over the same 133120 x 16384 tensor with its
    largest magnitude (-8192) planted at the very last element, past 2^31
    elements: the amax pass finds it, the tensor scale is amax / 43008, and
    sampled rows of both orientations (the planted element's row and column
    among them) are bit-exact with the oracle."""
    import torch

    block, x = big_x
    old = x[R - 1, C - 1].clone()
    x[R - 1, C - 1] = np.int16(np.uint16(0xC600).view(np.int16))  # bf16 -8192
    try:
        ts, amax = dev_scalar(1.0), dev_scalar(0.0)
        qr, qc = lib.empty_quantized(R, C, ts), lib.empty_quantized(C, R, ts)
        lib.quantize_current_scaling(x, ts, amax, lib.RNE, row=qr, col=qc)
        torch.cuda.synchronize()
        assert host(amax)[0] == np.float32(8192.0)
        ts_val = np.float32(np.float32(8192.0) / np.float32(6.0 * 7168.0))
        assert host(ts)[0] == ts_val
        rows_bits = block[ROWS % PERIOD].copy()
        rows_bits[-1, C - 1] = 0xC600  # ROWS ends with R - 1
        c, s_ = quantize.quantize_blockscale(rows_bits, ts_val, quantize.RNE)
        assert np.array_equal(host(qr.codes[ROWS.tolist()]), c) and np.array_equal(host(qr.scales[ROWS.tolist()]), s_)
        cols = np.tile(block[:, [0, C - 1]], (-(-R // PERIOD), 1))[:R].copy()
        cols[R - 1, 1] = 0xC600
        c, s_ = quantize.quantize_blockscale(cols, ts_val, quantize.RNE, orientation=1)
        assert np.array_equal(host(qc.codes[[0, C - 1]]), c) and np.array_equal(host(qc.scales[[0, C - 1]]), s_)
        del qr, qc
    finally:
        x[R - 1, C - 1] = old
        torch.cuda.synchronize()


def test_gemm_output_past_2_31_entries(cuda_device):
    import torch

    M, N, K = 65536, 36864, 32
    rng = np.random.default_rng(9)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    asc = rng.integers(0x60, 0x90, size=(M, K // 16), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bsc = rng.integers(0x60, 0x90, size=(N, K // 16), dtype=np.uint8)
    a = lib.Quantized(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(0.5))
    b = lib.Quantized(torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(0.25))
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    assert c.numel() > 2**31
    lib.gemm_nt(a, b, c)
    rows = np.array([0, 1, 30000, 58254, 65535, 65535, 40000, 65535])
    cols = np.array([0, 36863, 17, 36000, 0, 36863, 12345, 36000])
    got = host(c[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
    from oracle import gemm as ogemm

    ref, bound = ogemm.gemm_nt_entries(ac, asc, 0.5, bc, bsc, 0.25, rows, cols)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5 * bound)
    del c
    torch.cuda.empty_cache()


def test_mxfp4_gemm_output_past_2_31_entries(cuda_device):
    """The native MXFP4 GEMM with an output past 2^31 entries: sampled
    entries against the oracle, every entry written (NaN-prefilled, checked
    finite band by band)."""
    import torch
    from oracle import mxfp4

    M, N, K = 65536, 36864, 32
    rng = np.random.default_rng(10)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, size=(M, K // 32), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bsc = rng.integers(110, 140, size=(N, K // 32), dtype=np.uint8)
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    assert c.numel() > 2**31
    lib.gemm_nt_mxfp4(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(0.5),
                      torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(0.25), c)
    rows = np.array([0, 1, 30000, 58254, 65535, 65535, 40000, 65535])
    cols = np.array([0, 36863, 17, 36000, 0, 36863, 12345, 36000])
    got = host(c[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()]).astype(np.float64)
    ref, bound = mxfp4.gemm_nt_mx(ac[rows], asc[rows], 0.5, bc[cols], bsc[cols], 0.25)
    ref, bound = np.diag(ref), np.diag(bound)
    assert np.all(np.abs(got - ref) <= 1e-5 * bound)
    for r in range(0, M, 8192):
        assert bool(torch.isfinite(c[r:r + 8192]).all()), f"unwritten or non-finite entries in rows {r}.."
    del c
    torch.cuda.empty_cache()


def test_dequantize_past_2_31_elements(cuda_device):
    """Dequantize of a 65536 x 32784 operand (past 2^31 elements): sampled
    rows bit-exact with the oracle's decode."""
    import torch
    from oracle import quantize as oq

    R, C = 65536, 32784
    rng = np.random.default_rng(11)
    codes = torch.randint(0, 256, (R, C // 2), dtype=torch.uint8, device="cuda")
    scales = torch.randint(0x01, 0xFF, (R, C // 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, C), dtype=torch.float32, device="cuda")
    assert out.numel() > 2**31
    lib.dequantize(lib.Quantized(codes, scales, dev_scalar(0.375)), out)
    rows = np.unique(np.concatenate([[0, 1, R - 1], rng.integers(0, R, size=5)]))
    idx = torch.from_numpy(rows).cuda()
    want = oq.dequantize(host(codes[idx]), host(scales[idx]), np.float32(0.375))
    assert np.array_equal(host(out[idx]).view(np.uint32), want.astype(np.float32).view(np.uint32))
    del out, codes, scales
    torch.cuda.empty_cache()


def test_gemm_bf16_output_past_2_31_entries(cuda_device):
    """The bf16 + amax epilogue with an output past 2^31 entries, on
    exact-sum operands (payloads 0, +-0.5, +-1; scales in [1, 1.875];
    power-of-two tensor scales): sampled entries bit-exact with the oracle's
    rounding of the exact C, every entry written (NaN-prefilled)."""
    import torch
    from oracle import formats
    from oracle import gemm as og

    M, N, K = 65536, 36864, 32
    rng = np.random.default_rng(12)

    def exact(rows):
        nib = rng.choice(np.array([0, 1, 2, 8, 9, 10], dtype=np.uint8), size=(rows, K))
        return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8), \
            rng.integers(0x78, 0x80, size=(rows, K // 16), dtype=np.uint8)

    ac, asc = exact(M)
    bc, bsc = exact(N)
    a = lib.Quantized(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(0.5))
    b = lib.Quantized(torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(0.25))
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert y.numel() > 2**31
    lib.gemm_nt_bf16(a, b, y, amax=dev_scalar(0.0))
    rows = np.array([0, 1, 30000, 58254, 65535, 65535, 40000, 65535])
    cols = np.array([0, 36863, 17, 36000, 0, 36863, 12345, 36000])
    ref, _ = og.gemm_nt(ac[rows], asc[rows], 0.5, bc[cols], bsc[cols], 0.25)
    ref = np.diag(ref) + 0.0
    want = formats.f32_to_bf16_rne(ref.astype(np.float32))
    got = host(y.view(torch.int16)[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()]).view(np.uint16)
    assert np.array_equal(got, want)
    for r in range(0, M, 8192):
        assert bool(torch.isfinite(y[r:r + 8192]).all()), f"unwritten entries in rows {r}.."
    del y
    torch.cuda.empty_cache()


# Past 2^35 elements the stochastic-rounding call numbers (element index / 8)
# no longer fit 32 bits: the kernels take the 64-bit counter form there.
# x is a generator block of BR x BC tiled on the device to R35 x C35
# (3.49e10 elements, 69.8 GB; outputs 19.6 GB per orientation).  Sampled
# output rows lie on both sides of the first call number with a nonzero high
# word (row 131072 of the row-wise output, column 258112 of the transposed
# one) and are compared with the oracle's row step on their own data and
# true coordinates.
R35, C35 = 133120, 262144
BR, BC = 1021, 8208
ROWS35 = [0, 1, 131071, 131072, 131073, R35 - 1]
COLS35 = [0, 7, 258111, 258112, 258113, C35 - 1]


@pytest.fixture(scope="module")
def big35(cuda_device):
    import torch

    assert R35 * C35 > 2**35 and (R35 * C35 - 8) // 8 >= 2**32
    block = random_bf16((BR, BC), seed=20261)
    wide = dev_bf16(block).repeat(1, -(-C35 // BC))[:, :C35].contiguous()  # BR x C35
    x = torch.empty((R35, C35), dtype=torch.int16, device="cuda")
    for r in range(0, R35, BR):
        x[r:r + BR] = wide[:min(BR, R35 - r)]
    del wide
    ts_val = np.float32(np.float32(quantize.tensor_amax(block)) / np.float32(43008.0))
    yield block, x, ts_val
    del x
    torch.cuda.empty_cache()


def test_stochastic_rounding_past_2_35_elements(big35):
    import torch
    from oracle import formats

    block, x, ts_val = big35
    ts = dev_scalar(ts_val)
    seed, offset = 0x1234_5678_9ABC_DEF0, 77
    qr = lib.empty_quantized(R35, C35, ts)
    qc = lib.empty_quantized(C35, R35, ts)
    lib.quantize_blockscale(x, ts, lib.SR, seed, offset, row=qr, col=qc)
    torch.cuda.synchronize()
    rows = np.array(ROWS35, dtype=np.int64)
    cols = np.array(COLS35, dtype=np.int64)
    # output rows of orientation 0: rows of x; of orientation 1: columns of x
    xr = block[rows % BR][:, np.arange(C35) % BC]
    xc = block[:, cols % BC][np.arange(R35) % BR].T
    for orient, data, ids, q in ((0, xr, rows, qr), (1, xc, cols, qc)):
        c, s = quantize._quantize_rows(formats.bf16_to_f32(data), ts_val, quantize.SR, seed, offset, orient,
                                       data.shape[1], ids)
        assert np.array_equal(host(q.scales[ids.tolist()]), s), f"scales, orientation {orient}"
        assert np.array_equal(host(q.codes[ids.tolist()]), c), f"codes, orientation {orient}"
    del qr, qc
    torch.cuda.empty_cache()


def test_stochastic_rounding_2d_past_2_35_elements(big35):
    import torch

    block, x, ts_val = big35
    ts = dev_scalar(ts_val)
    seed, offset = 0x0FED_CBA9_8765_4321, 5
    qr = lib.empty_quantized(R35, C35, ts)
    qc = lib.empty_quantized(C35, R35, ts)
    lib.quantize_blockscale_2d(x, ts, lib.SR, seed, offset, row=qr, col=qc)
    torch.cuda.synchronize()
    # 16-row groups: 8191 ends just below the first call number past 2^32
    # (row 131072), 8192 starts there
    for g in (0, 8191, 8192, R35 // 16 - 1):
        xs = block[(16 * g + np.arange(16)) % BR][:, np.arange(C35) % BC]
        rc, rs, cc, cs, _ = quantize2d.quantize_blockscale_2d(xs, ts_val, quantize.SR, seed, offset, row0=16 * g)
        assert np.array_equal(host(qr.codes[16 * g:16 * g + 16]), rc), f"row codes, group {g}"
        assert np.array_equal(host(qr.scales[16 * g:16 * g + 16]), rs), f"row scales, group {g}"
        assert np.array_equal(host(qc.codes[:, 8 * g:8 * g + 8]), cc), f"col codes, group {g}"
        assert np.array_equal(host(qc.scales[:, g:g + 1]), cs), f"col scales, group {g}"
    del qr, qc
    torch.cuda.empty_cache()

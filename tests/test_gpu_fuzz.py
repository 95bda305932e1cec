"""Seeded randomized parity cases: each case draws its own parameter mix
from its index, so combinations the targeted tests cover one at a time meet
here -- ragged and strided inputs, NaN / Inf / signed-zero elements and
all-zero blocks, tensor scales off the fresh value by non-power-of-two
factors and special ones (0, Inf, NaN, negative, 1e-45, 3e38), both
roundings with 64-bit seeds and 32-bit offsets, every output combination,
the amax by-product, current-tensor scaling with random max_safe, GEMMs
over random codes with 0x00 / 0xFF scales, negative tensor scales and K
tails, and the quantizing GEMM epilogue on exact-sum operands.  Every output
is compared with the oracle: codes and scale bytes bit for bit, the amax and
tensor scale exactly, GEMM entries within 1e-5 |tsA tsB| sum|a b| with the
same NaN pattern, the epilogue's bf16 output bit for bit with the oracle's
rounding of the exact C.
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, mxfp4, quantize, quantize2d, tensor_scale
from oracle import gemm as ogemm

from devhelpers import assert_gemm_close, dev_scalar, host
from workloads import random_bf16

pytestmark = pytest.mark.gpu

KINDS = ("normal", "heavy", "logrange", "gradient")
SPECIAL_TS = (0.0, np.inf, -np.inf, np.nan, -1.0, 1e-45, 3e38)


def _input(rng, rows, cols):
    """bf16 bits of a random kind, with specials sprinkled in some cases."""
    kind = KINDS[rng.integers(len(KINDS))]
    bits = random_bf16((rows, cols), int(rng.integers(1 << 31)), kind)
    if rng.random() < 0.35:
        n = int(rng.integers(1, 6))
        r, c = rng.integers(rows, size=n), rng.integers(cols, size=n)
        bits[r, c] = rng.choice(np.array([0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001], dtype=np.uint16), size=n)
    if rng.random() < 0.35:
        r, b = int(rng.integers(rows)), int(rng.integers(cols // 16))
        bits[r, 16 * b:16 * b + 16] = 0
    return kind, bits


def _tensor_scale(rng, bits):
    """A tensor scale near the fresh one (finite part's amax / 43008) times a
    random non-power-of-two factor, or a special value."""
    if rng.random() < 0.12:
        return np.float32(SPECIAL_TS[rng.integers(len(SPECIAL_TS))])
    x = np.abs(formats.bf16_to_f32(bits).astype(np.float64))
    x = x[np.isfinite(x)]
    amax = float(x.max()) if x.size and x.max() > 0 else 1.0
    return np.float32(amax / 43008.0 * 2.0 ** int(rng.integers(-6, 7)) * (1.0 + rng.random()))


def _device_strided(bits, pad):
    """The bits on the device as the first `cols` columns of a wider tensor
    (row stride cols + pad)."""
    import torch

    rows, cols = bits.shape
    full = np.zeros((rows, cols + pad), dtype=np.uint16)
    full[:, :cols] = bits
    return torch.from_numpy(full.view(np.int16)).cuda()[:, :cols]


def _check_amax(got, bits):
    want = quantize.tensor_amax(bits)
    if np.isnan(want):
        assert np.isnan(got), "amax should be NaN"
    else:
        assert got == want, f"amax {got!r} != {want!r}"


def _check(q, oracle_codes, oracle_scales, what):
    gc, gs = host(q.codes), host(q.scales)
    bad = np.argwhere(gs != oracle_scales)
    assert bad.size == 0, f"{what}: scales differ at {bad[:4].tolist()}"
    bad = np.argwhere(gc != oracle_codes)
    assert bad.size == 0, f"{what}: codes differ at {bad[:4].tolist()}"


@pytest.mark.parametrize("case", range(80))
def test_quantize_random_case(cuda_device, case):
    import torch

    rng = np.random.default_rng(7_000 + case)
    want_col = rng.random() < 0.6
    rows = 16 * int(rng.integers(1, 26)) if want_col else int(rng.integers(1, 420))
    cols = 16 * int(rng.integers(1, 42))
    pad = 8 * int(rng.integers(0, 4))
    want_row = (not want_col) or rng.random() < 0.7
    kind, bits = _input(rng, rows, cols)
    ts = _tensor_scale(rng, bits)
    rounding = lib.SR if rng.random() < 0.5 else lib.RNE
    seed, offset = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(2)), int(rng.integers(0, 2**32))
    use_amax = rng.random() < 0.5
    desc = (f"case {case}: {rows}x{cols} ld+{pad} {kind} ts={ts!r} "
            f"{'SR' if rounding else 'RNE'} seed={seed:#x} offset={offset} row={want_row} col={want_col}")
    x = _device_strided(bits, pad)
    ts_dev = dev_scalar(ts)
    qr = lib.empty_quantized(rows, cols, ts_dev) if want_row else None
    qc = lib.empty_quantized(cols, rows, ts_dev) if want_col else None
    amax = torch.zeros(1, dtype=torch.float32, device="cuda") if use_amax else None
    lib.quantize_blockscale(x, ts_dev, rounding, seed, offset, row=qr, col=qc, amax=amax)
    for q, o in ((qr, 0), (qc, 1)):
        if q is not None:
            oc, os_ = quantize.quantize_blockscale(bits, ts, rounding, seed, offset, o)
            _check(q, oc, os_, f"{desc}, orientation {o}")
    if use_amax:
        _check_amax(host(amax)[0], bits)


@pytest.mark.parametrize("case", range(30))
def test_quantize_2d_random_case(cuda_device, case):
    rng = np.random.default_rng(8_000 + case)
    rows, cols = 16 * int(rng.integers(1, 22)), 16 * int(rng.integers(1, 42))
    pad = 8 * int(rng.integers(0, 4))
    want_row, want_col = [(True, True), (True, False), (False, True)][int(rng.integers(3))]
    kind, bits = _input(rng, rows, cols)
    ts = _tensor_scale(rng, bits)
    rounding = lib.SR if rng.random() < 0.5 else lib.RNE
    seed, offset = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    desc = f"case {case}: {rows}x{cols} ld+{pad} {kind} ts={ts!r} {'SR' if rounding else 'RNE'} seed={seed:#x}"
    x = _device_strided(bits, pad)
    ts_dev = dev_scalar(ts)
    qr = lib.empty_quantized(rows, cols, ts_dev) if want_row else None
    qc = lib.empty_quantized(cols, rows, ts_dev) if want_col else None
    lib.quantize_blockscale_2d(x, ts_dev, rounding, seed, offset, row=qr, col=qc)
    rc, rs, cc, cs, _ = quantize2d.quantize_blockscale_2d(bits, ts, rounding, seed, offset)
    if qr is not None:
        _check(qr, rc, rs, f"{desc}, row-wise")
    if qc is not None:
        _check(qc, cc, cs, f"{desc}, transposed")


def _random_operand(rng, rows, k, block):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    lo, hi = (0x01, 0xFF) if block == 16 else (100, 150)
    scales = rng.integers(lo, hi, size=(rows, k // block), dtype=np.uint8)
    if block == 16 and scales.size and rng.random() < 0.4:
        n = int(rng.integers(1, 4))
        scales.flat[rng.integers(scales.size, size=n)] = rng.choice(np.array([0x00, 0xFF], dtype=np.uint8), size=n)
    return codes, scales


def _random_ts(rng):
    return np.float32((-1.0 if rng.random() < 0.2 else 1.0) * 2.0 ** rng.uniform(-20, 10))


@pytest.mark.parametrize("case", range(40))
def test_gemm_random_case(cuda_device, case):
    import torch

    rng = np.random.default_rng(9_000 + case)
    M, N = int(rng.integers(1, 620)), int(rng.integers(1, 620))
    K = 16 * int(rng.integers(0, 70))
    ac, asc = _random_operand(rng, M, K, 16)
    bc, bsc = _random_operand(rng, N, K, 16)
    ta, tb = _random_ts(rng), _random_ts(rng)
    a = lib.Quantized(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(ta))
    b = lib.Quantized(torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(tb))
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lib.gemm_nt(a, b, c)
    assert_gemm_close(host(c), ac, asc, ta, bc, bsc, tb)


@pytest.mark.parametrize("case", range(16))
def test_gemm_mxfp4_random_case(cuda_device, case):
    import torch

    rng = np.random.default_rng(9_500 + case)
    M, N = int(rng.integers(1, 620)), int(rng.integers(1, 620))
    K = 32 * int(rng.integers(1, 40))
    ac, asc = _random_operand(rng, M, K, 32)
    bc, bsc = _random_operand(rng, N, K, 32)
    ta, tb = _random_ts(rng), _random_ts(rng)
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lib.gemm_nt_mxfp4(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(ta),
                      torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(tb), c)
    got = host(c).astype(np.float64)
    ref, bound = mxfp4.gemm_nt_mx(ac, asc, ta, bc, bsc, tb)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.all(np.abs(got - ref)[ok] <= 1e-5 * bound[ok])


@pytest.mark.parametrize("case", range(24))
def test_current_scaling_random_case(cuda_device, case):
    rng = np.random.default_rng(10_000 + case)
    want_row, want_col = [(True, True), (True, False), (False, True)][int(rng.integers(3))]
    rows = 16 * int(rng.integers(1, 26)) if want_col else int(rng.integers(1, 420))
    cols, pad = 16 * int(rng.integers(1, 42)), 8 * int(rng.integers(0, 4))
    kind, bits = _input(rng, rows, cols)
    if rng.random() < 0.1:
        bits[:] = 0
    rounding = lib.SR if rng.random() < 0.5 else lib.RNE
    seed, offset = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    max_safe = np.float32(7168.0 if rng.random() < 0.5 else rng.uniform(1.0, 114688.0))
    ts_prev = np.float32(2.0 ** rng.uniform(-20, 4))
    desc = f"case {case}: {rows}x{cols} ld+{pad} {kind} max_safe={max_safe!r} {'SR' if rounding else 'RNE'}"
    amax_ref = quantize.tensor_amax(bits)
    _, ts_ref = tensor_scale.update_tensor_scale(amax_ref, ts_prev, 0, 1, max_safe)
    x = _device_strided(bits, pad)
    ts_dev, amax_dev = dev_scalar(ts_prev), dev_scalar(123.0)
    qr = lib.empty_quantized(rows, cols, ts_dev) if want_row else None
    qc = lib.empty_quantized(cols, rows, ts_dev) if want_col else None
    lib.quantize_current_scaling(x, ts_dev, amax_dev, rounding, seed, offset, row=qr, col=qc, max_safe=float(max_safe))
    _check_amax(host(amax_dev)[0], bits)
    assert host(ts_dev)[0].tobytes() == ts_ref.tobytes(), f"{desc}: tensor scale"
    for q, o in ((qr, 0), (qc, 1)):
        if q is not None:
            oc, os_ = quantize.quantize_blockscale(bits, ts_ref, rounding, seed, offset, o)
            _check(q, oc, os_, f"{desc}, orientation {o}")


EXACT_CODES = np.array([0, 1, 2, 8, 9, 10], dtype=np.uint8)  # 0, 0.5, 1 and their negatives


def _exact_operand(rng, rows, k, ts):
    """Payload magnitudes <= 1, scales in [1, 1.875] and a power-of-two
    tensor scale: every fp32 partial sum of the GEMM is exact (K <= 4112)."""
    import torch

    nib = rng.choice(EXACT_CODES, size=(rows, k))
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0x78, 0x80, size=(rows, k // 16), dtype=np.uint8)
    q = lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), dev_scalar(ts))
    return q, codes, scales


@pytest.mark.parametrize("case", range(24))
def test_quantizing_epilogue_random_case(cuda_device, case):
    import torch

    rng = np.random.default_rng(11_000 + case)
    M, N, K = 16 * int(rng.integers(1, 40)), 16 * int(rng.integers(1, 40)), 16 * int(rng.integers(0, 70))
    ta = np.float32((-1.0 if rng.random() < 0.3 else 1.0) * 2.0 ** int(rng.integers(-10, 5)))
    tb = np.float32(2.0 ** int(rng.integers(-10, 5)))
    a, ac, asc = _exact_operand(rng, M, K, ta)
    b, bc, bsc = _exact_operand(rng, N, K, tb)
    ref, _ = ogemm.gemm_nt(ac, asc, ta, bc, bsc, tb)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref), "operands do not give exact sums"
    # An exact zero sum is +0 in the fp32 accumulators; the epilogue's
    # products (acc * 256 tsA) * tsB give it the sign of tsA * tsB.
    ref = np.where(ref == 0.0, np.copysign(0.0, float(ta) * float(tb)), ref)
    ybits = formats.f32_to_bf16_rne(ref.astype(np.float32))
    out_ts = _tensor_scale(rng, ybits)
    rounding = lib.SR if rng.random() < 0.5 else lib.RNE
    seed, offset = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    want_row, want_col = [(True, True), (True, False), (False, True)][int(rng.integers(3))]
    desc = f"case {case}: {M}x{N}x{K} out_ts={out_ts!r} {'SR' if rounding else 'RNE'} row={want_row} col={want_col}"
    ts_dev = dev_scalar(out_ts)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    qr = lib.empty_quantized(M, N, ts_dev) if want_row else None
    qc = lib.empty_quantized(N, M, ts_dev) if want_col else None
    lib.gemm_nt_bf16_quantized(a, b, y, ts_dev, rounding, seed, offset, row=qr, col=qc, amax=amax)
    got = host(y.view(torch.int16)).view(np.uint16)
    assert np.array_equal(got, ybits), f"{desc}: bf16 output"
    _check_amax(host(amax)[0], ybits)
    for q, o in ((qr, 0), (qc, 1)):
        if q is not None:
            oc, os_ = quantize.quantize_blockscale(ybits, out_ts, rounding, seed, offset, o)
            _check(q, oc, os_, f"{desc}, orientation {o}")


@pytest.mark.parametrize("case", range(16))
def test_exact_sum_outputs_random_case(cuda_device, case):
    """fp32 and bf16 (+ amax) outputs on exact-sum operands, ragged M and N,
    tensor scales of either sign: bit for bit, zero signs included (R20)."""
    import torch

    rng = np.random.default_rng(12_000 + case)
    M, N, K = int(rng.integers(1, 620)), int(rng.integers(1, 620)), 16 * int(rng.integers(0, 70))
    ta = np.float32((-1.0 if rng.random() < 0.4 else 1.0) * 2.0 ** int(rng.integers(-10, 5)))
    tb = np.float32((-1.0 if rng.random() < 0.4 else 1.0) * 2.0 ** int(rng.integers(-10, 5)))
    a, ac, asc = _exact_operand(rng, M, K, ta)
    b, bc, bsc = _exact_operand(rng, N, K, tb)
    ref, _ = ogemm.gemm_nt(ac, asc, ta, bc, bsc, tb)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref), "operands do not give exact sums"
    ref = np.where(ref == 0.0, np.copysign(0.0, float(ta) * float(tb)), ref).astype(np.float32)
    desc = f"case {case}: {M}x{N}x{K} ta={ta!r} tb={tb!r}"
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lib.gemm_nt(a, b, c)
    bad = np.argwhere(host(c).view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"{desc}: fp32 output differs at {bad[:4].tolist()}"
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    lib.gemm_nt_bf16(a, b, y, amax=amax)
    ybits = formats.f32_to_bf16_rne(ref)
    got = host(y.view(torch.int16)).view(np.uint16)
    bad = np.argwhere(got != ybits)
    assert bad.size == 0, f"{desc}: bf16 output differs at {bad[:4].tolist()}"
    _check_amax(host(amax)[0], ybits)


@pytest.mark.parametrize("case", range(8))
def test_gemm_multi_tile_random_case(cuda_device, case):
    """Random sizes past the 8-tile threshold of the XCD-remapped tile order
    (up to 13 x 13 tiles, ragged tile-row groups and edges): whole output."""
    import torch

    rng = np.random.default_rng(13_000 + case)
    M, N = int(rng.integers(257, 3300)), int(rng.integers(257, 3300))
    K = 16 * int(rng.integers(1, 40))
    ac, asc = _random_operand(rng, M, K, 16)
    bc, bsc = _random_operand(rng, N, K, 16)
    ta, tb = _random_ts(rng), _random_ts(rng)
    a = lib.Quantized(torch.from_numpy(ac).cuda(), torch.from_numpy(asc).cuda(), dev_scalar(ta))
    b = lib.Quantized(torch.from_numpy(bc).cuda(), torch.from_numpy(bsc).cuda(), dev_scalar(tb))
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lib.gemm_nt(a, b, c)
    assert_gemm_close(host(c), ac, asc, ta, bc, bsc, tb)


@pytest.mark.parametrize("case", range(8))
def test_quantize_multi_tile_random_case(cuda_device, case):
    """Random sizes of many tiles (the quantizer's XCD-grouped band order),
    both outputs, strided input."""
    rng = np.random.default_rng(14_000 + case)
    rows, cols = 16 * int(rng.integers(20, 130)), 16 * int(rng.integers(20, 260))
    pad = 8 * int(rng.integers(0, 4))
    kind, bits = _input(rng, rows, cols)
    ts = _tensor_scale(rng, bits)
    rounding = lib.SR if rng.random() < 0.5 else lib.RNE
    seed, offset = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    desc = f"case {case}: {rows}x{cols} ld+{pad} {kind} ts={ts!r} {'SR' if rounding else 'RNE'}"
    x = _device_strided(bits, pad)
    ts_dev = dev_scalar(ts)
    qr, qc = lib.empty_quantized(rows, cols, ts_dev), lib.empty_quantized(cols, rows, ts_dev)
    lib.quantize_blockscale(x, ts_dev, rounding, seed, offset, row=qr, col=qc)
    for q, o in ((qr, 0), (qc, 1)):
        oc, os_ = quantize.quantize_blockscale(bits, ts, rounding, seed, offset, o)
        _check(q, oc, os_, f"{desc}, orientation {o}")

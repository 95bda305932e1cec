"""GPU parity of the quantizer (HIP kernels through the C ABI) with the oracle.

Codes and scale bytes must match bit-exactly, in both rounding modes and both
output orientations ("UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", abstract: block-16 E2M1/UE5M3 under a tensor scale, stochastic
rounding on gradients).
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, quantize, tensor_scale
from workloads import config, random_bf16, sr_seed, to_bf16_bits, STALE_FACTORS

from devhelpers import (assert_quant_equal, dev_bf16, dev_scalar, fresh_ts, gpu_quantize, host,
                        oracle_operand, sample_rows)

pytestmark = pytest.mark.gpu

MODES = [(lib.RNE, "rne"), (lib.SR, "sr")]


@pytest.mark.parametrize("rounding,name", MODES)
@pytest.mark.parametrize("shape,kind", [((256, 256), "normal"), ((144, 544), "heavy"),
                                        ((400, 48), "gradient"), ((16, 16), "normal"),
                                        ((1024, 1040), "logrange")])
def test_quantize_full_compare(cuda_device, rounding, name, shape, kind):
    """Whole outputs compared: several workgroup tiles plus ragged tails."""
    bits = random_bf16(shape, seed=sum(shape), kind=kind)
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    amax = dev_scalar(0.0)
    qr, qc = gpu_quantize(x, ts, rounding, seed=99, offset=3, amax=amax)
    assert_quant_equal(qr, bits, ts, rounding, 99, 3, 0)
    assert_quant_equal(qc, bits, ts, rounding, 99, 3, 1)
    assert host(amax)[0] == quantize.tensor_amax(bits)


@pytest.mark.parametrize("rows", [1, 5, 17, 130, 300])
def test_row_only_ragged_rows(cuda_device, rows):
    """Row-wise output alone allows any row count."""
    bits = random_bf16((rows, 272), seed=rows)
    ts = fresh_ts(bits)
    for rounding, _ in MODES:
        qr, _ = gpu_quantize(dev_bf16(bits), ts, rounding, seed=7, offset=1, col=False)
        assert_quant_equal(qr, bits, ts, rounding, 7, 1, 0)


def test_col_only_and_row_only_agree_with_fused(cuda_device):
    bits = random_bf16((256, 512), seed=31, kind="heavy")
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    for rounding, _ in MODES:
        qr, qc = gpu_quantize(x, ts, rounding, seed=5, offset=9)
        qr1, _ = gpu_quantize(x, ts, rounding, seed=5, offset=9, col=False)
        _, qc1 = gpu_quantize(x, ts, rounding, seed=5, offset=9, row=False)
        assert np.array_equal(host(qr.codes), host(qr1.codes))
        assert np.array_equal(host(qr.scales), host(qr1.scales))
        assert np.array_equal(host(qc.codes), host(qc1.codes))
        assert np.array_equal(host(qc.scales), host(qc1.scales))


def test_strided_input(cuda_device):
    """A row stride (ld) larger than the width: a column slice of a wider tensor."""
    import torch

    wide = random_bf16((64, 320), seed=41)
    x = dev_bf16(wide)[:, 32:288]
    bits = np.ascontiguousarray(wide[:, 32:288])
    assert x.stride(0) == 320
    ts = fresh_ts(bits)
    qr, qc = gpu_quantize(x, ts, lib.SR, seed=1, offset=2)
    assert_quant_equal(qr, bits, ts, lib.SR, 1, 2, 0)
    assert_quant_equal(qc, bits, ts, lib.SR, 1, 2, 1)


def test_amax_only_pass_and_running_max(cuda_device):
    bits = random_bf16((300, 64), seed=2, kind="heavy")
    amax = dev_scalar(0.0)
    lib.quantize_blockscale(dev_bf16(bits), None, amax=amax)
    assert host(amax)[0] == quantize.tensor_amax(bits)
    # running max: a larger prior value survives, a smaller one is replaced
    amax = dev_scalar(1e30)
    lib.quantize_blockscale(dev_bf16(bits), None, amax=amax)
    assert host(amax)[0] == np.float32(1e30)


def test_empty_input_is_a_no_op(cuda_device):
    import torch

    x = torch.zeros((0, 32), dtype=torch.int16, device="cuda")
    amax = dev_scalar(0.5)
    qr = lib.empty_quantized(0, 32, dev_scalar(1.0))
    lib.quantize_blockscale(x, qr.ts, lib.RNE, row=qr, amax=amax)
    assert host(amax)[0] == np.float32(0.5)


def test_nonfinite_inputs_and_degenerate_scales(cuda_device):
    x = np.ones((32, 64), dtype=np.float32)
    x[0, 3] = np.inf
    x[17, 40] = np.nan
    x[5, 5] = -np.inf
    from workloads import to_bf16_bits

    bits = to_bf16_bits(x)
    for ts in (np.float32(1.0), np.float32(0.0), np.float32(np.inf), np.float32(-2.0),
               np.float32(np.nan), np.float32(1e-38)):
        for rounding, _ in MODES:
            qr, qc = gpu_quantize(dev_bf16(bits), ts, rounding, seed=3)
            assert_quant_equal(qr, bits, ts, rounding, 3, 0, 0)
            assert_quant_equal(qc, bits, ts, rounding, 3, 0, 1)
    amax = dev_scalar(0.0)
    lib.quantize_blockscale(dev_bf16(bits), None, amax=amax)
    assert np.isnan(host(amax)[0])


def test_tiny_tensor_scale_overflowing_reciprocal(cuda_device):
    """ts * s_b underflows so 1 / (ts * s_b) is +Inf: nonzero elements
    saturate, zeros stay zero (a NaN product encodes magnitude 0)."""
    x = np.zeros((16, 32), dtype=np.float32)
    x[:, 0] = 1e-38
    x[:, 1] = -3e-39
    from workloads import to_bf16_bits

    bits = to_bf16_bits(x)
    for ts in (np.float32(1e-45), np.float32(3e-44)):
        for rounding, _ in MODES:
            qr, qc = gpu_quantize(dev_bf16(bits), ts, rounding, seed=8)
            assert_quant_equal(qr, bits, ts, rounding, 8, 0, 0)
            assert_quant_equal(qc, bits, ts, rounding, 8, 0, 1)


@pytest.mark.parametrize("rounding,name", MODES)
def test_config2_activations(cuda_device, rounding, name):
    """8192 x 4096 heavy-tailed activations with outlier columns: both
    orientations, sampled rows compared with the oracle; the row-wise output
    of the fused call equals the row-only call everywhere."""
    bits = config(2)["X"]
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    amax = dev_scalar(0.0)
    qr, qc = gpu_quantize(x, ts, rounding, seed=sr_seed(2), offset=0, amax=amax)
    assert host(amax)[0] == quantize.tensor_amax(bits)
    assert_quant_equal(qr, bits, ts, rounding, sr_seed(2), 0, 0, rows=sample_rows(8192, 96, 1))
    assert_quant_equal(qc, bits, ts, rounding, sr_seed(2), 0, 1, rows=sample_rows(4096, 48, 2))
    qr1, _ = gpu_quantize(x, ts, rounding, seed=sr_seed(2), offset=0, col=False)
    assert np.array_equal(host(qr.codes), host(qr1.codes))
    assert np.array_equal(host(qr.scales), host(qr1.scales))


@pytest.mark.parametrize("factor", STALE_FACTORS)
def test_config5_stale_scale(cuda_device, factor):
    """Dynamic-range stress with a tensor scale from an amax off by x8 or x1/8:
    no block saturates, codes bit-exact on sampled rows, flushed-block counts
    match the oracle's definition."""
    data = config(5)
    for name, rounding in (("X", lib.RNE), ("W", lib.RNE), ("dY", lib.SR)):
        bits = data[name]
        amax = quantize.tensor_amax(bits)
        _, ts = tensor_scale.update_tensor_scale(np.float32(amax * np.float32(factor)),
                                                 np.float32(1.0), 0, 1)
        qr, qc = gpu_quantize(dev_bf16(bits), ts, rounding, seed=sr_seed(5), offset=1)
        assert_quant_equal(qr, bits, ts, rounding, sr_seed(5), 1, 0, rows=sample_rows(4096, 32, 3))
        assert_quant_equal(qc, bits, ts, rounding, sr_seed(5), 1, 1, rows=sample_rows(4096, 32, 4))
        s = host(qr.scales)
        assert not np.any(s == 0xFF)
        x = formats.bf16_to_f32(bits)
        amax_b = np.abs(x).reshape(4096, 256, 16).max(axis=2)
        s_raw = amax_b / (np.float32(6) * ts)
        assert np.all(s_raw <= formats.UE5M3_MAX)  # nothing saturates
        assert np.array_equal(s == 0, formats.ue5m3_encode(s_raw) == 0)


def test_deterministic(cuda_device):
    bits = random_bf16((512, 1024), seed=77, kind="gradient")
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    a = gpu_quantize(x, ts, lib.SR, seed=4, offset=4)
    b = gpu_quantize(x, ts, lib.SR, seed=4, offset=4)
    for qa, qb in zip(a, b):
        assert np.array_equal(host(qa.codes), host(qb.codes))
        assert np.array_equal(host(qa.scales), host(qb.scales))


def test_dequantize_bit_exact(cuda_device):
    import torch

    bits = random_bf16((144, 512), seed=12, kind="logrange")
    ts = fresh_ts(bits)
    qr, qc = gpu_quantize(dev_bf16(bits), ts, lib.SR, seed=2)
    for o, q in enumerate((qr, qc)):
        oc, os_ = oracle_operand(bits, ts, lib.SR, 2, 0, o, q_gpu=q)  # the GPU's codes are the oracle's
        out = torch.empty((q.rows, q.cols), dtype=torch.float32, device="cuda")
        lib.dequantize(q, out)
        ref = quantize.dequantize(oc, os_, ts)
        got = host(out)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # NaN scale blocks dequantize to NaN
    q = lib.empty_quantized(16, 32, dev_scalar(2.0))
    q.codes.fill_(0x21)
    q.scales.fill_(0xFF)
    q.scales[3, 1] = 0x78
    out = torch.empty((16, 32), dtype=torch.float32, device="cuda")
    lib.dequantize(q, out)
    got = host(out)
    assert np.isnan(got).sum() == 16 * 32 - 16
    assert np.all(got[3, 16:] == np.float32(2.0) * formats.e2m1_decode(np.array([1, 2] * 8)))


def test_update_tensor_scale(cuda_device):
    for amax, ts, step, period in [(43008.0, 5.0, 0, 1), (7.0, 2.0, 8, 4), (7.0, 2.0, 9, 4),
                                   (0.0, 3.0, 0, 1), (np.nan, 3.0, 2, 2), (np.inf, 3.0, 0, 1),
                                   (1e-30, 1.0, 0, 1)]:
        a_dev, t_dev = dev_scalar(amax), dev_scalar(ts)
        lib.update_tensor_scale(a_dev, t_dev, step, period)
        ea, et = tensor_scale.update_tensor_scale(np.float32(amax), np.float32(ts), step, period)
        ga, gt = host(a_dev)[0], host(t_dev)[0]
        assert (ga == ea) or (np.isnan(ga) and np.isnan(ea))
        assert gt == et
    a_dev, t_dev = dev_scalar(3.0), dev_scalar(1.0)
    lib.update_tensor_scale(a_dev, t_dev, 0, 1, max_safe=0.5)
    assert host(t_dev)[0] == np.float32(1.0)


@pytest.mark.parametrize("rounding,name", MODES)
@pytest.mark.parametrize("shape,kind", [((272, 528), "heavy"), ((1024, 1040), "logrange"),
                                        ((64, 256), "zeros")])
def test_current_scaling(cuda_device, rounding, name, shape, kind):
    """Current-tensor scaling: the amax of this tensor, ts = amax / (6 max_safe)
    (the update rule applied to a fresh amax, ts kept when the amax is 0),
    then the same block quantization -- codes, scales, amax and ts bit-exact."""
    if kind == "zeros":
        bits = np.zeros(shape, dtype=np.uint16)
    else:
        bits = random_bf16(shape, seed=7 + shape[0], kind=kind)
    amax_ref = quantize.tensor_amax(bits)
    _, ts_ref = tensor_scale.update_tensor_scale(amax_ref, np.float32(0.5), 0, 1)
    x = dev_bf16(bits)
    ts_dev, amax_dev = dev_scalar(0.5), dev_scalar(123.0)
    rows, cols = shape
    qr, qc = lib.empty_quantized(rows, cols, ts_dev), lib.empty_quantized(cols, rows, ts_dev)
    lib.quantize_current_scaling(x, ts_dev, amax_dev, rounding, seed=5, offset=9, row=qr, col=qc)
    assert host(amax_dev)[0] == amax_ref
    assert host(ts_dev)[0] == ts_ref
    assert_quant_equal(qr, bits, ts_ref, rounding, 5, 9, 0)
    assert_quant_equal(qc, bits, ts_ref, rounding, 5, 9, 1)


@pytest.mark.parametrize("shape,ld,kind", [((48, 64), 64, "heavy"), ((37, 80), 96, "normal"),
                                           ((4096, 528), 528, "logrange"), ((3, 16), 24, "normal"),
                                           ((2048, 4096), 4096, "gradient")])
def test_amax_only_pass(cuda_device, shape, ld, kind):
    """The amax-only pass (bootstrap and current scaling): contiguous and
    strided rows, grid-stride tails, a running value that is already larger,
    and NaN propagation."""
    import torch

    rows, cols = shape
    bits = random_bf16(shape, seed=rows + ld, kind=kind)
    full = np.zeros((rows, ld), dtype=np.uint16)
    full[:, :cols] = bits
    full[:, cols:] = 0x7F80  # +Inf in the padding must not be read
    xd = torch.from_numpy(full.view(np.int16)).cuda()[:, :cols]
    amax = dev_scalar(0.0)
    lib.quantize_blockscale(xd, None, amax=amax)
    assert host(amax)[0] == quantize.tensor_amax(bits)
    big = dev_scalar(1e30)
    lib.quantize_blockscale(xd, None, amax=big)
    assert host(big)[0] == np.float32(1e30)
    bits2 = bits.copy()
    bits2[rows - 1, cols - 1] = 0x7FC0
    full[:, :cols] = bits2
    xd2 = torch.from_numpy(full.view(np.int16)).cuda()[:, :cols]
    nan_amax = dev_scalar(0.0)
    lib.quantize_blockscale(xd2, None, amax=nan_amax)
    assert np.isnan(host(nan_amax)[0])


def test_earlier_runtime_error_is_not_reported(cuda_device):
    """An error left in the runtime's per-thread last-error slot by an earlier,
    unrelated call (here a failed hipSetDevice) is not reported as the
    library's own launch failure."""
    import ctypes

    import torch

    bits = random_bf16((64, 64), seed=5)
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    ts_dev = dev_scalar(ts)
    qr, qc = lib.empty_quantized(64, 64, ts_dev), lib.empty_quantized(64, 64, ts_dev)
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so")
    assert hip.hipSetDevice(1 << 20) != 0  # invalid ordinal: fails, changes nothing
    st = lib.load_library().ue5m3fp4_quantize_blockscale(
        x.data_ptr(), 64, 64, 64, ts_dev.data_ptr(), lib.RNE, 0, 0, qr.codes.data_ptr(),
        qr.scales.data_ptr(), qc.codes.data_ptr(), qc.scales.data_ptr(), None, None)
    hip.hipGetLastError()  # leave the slot clean for the framework either way
    assert st == 0, lib.status_string(st)
    assert_quant_equal(qr, bits, ts, lib.RNE, 0, 0, 0)
    assert_quant_equal(qc, bits, ts, lib.RNE, 0, 0, 1)


@pytest.mark.parametrize("seed", [1, 77, 2**40 + 3])
def test_sr_every_magnitude_class(cuda_device, seed):
    """Stochastic rounding over scaled magnitudes from 6 down to 2^-24 (every
    E2M1 interval, the sub-2^-9 range, values on and next to grid points),
    both orientations, several random streams: bit-exact with the oracle."""
    rng = np.random.default_rng(seed % 1000)
    R, C = 128, 512
    u = rng.uniform(-24.0, 0.0, size=(R, C))
    x = np.sign(rng.standard_normal((R, C))) * np.exp2(u)
    x[:, ::16] = 1.0                                   # every row block: amax 1
    grid = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0]) / 6.0
    x[::3, 5::16] = rng.choice(grid, size=x[::3, 5::16].shape)  # near grid points
    bits = to_bf16_bits(x.astype(np.float32))
    ts = np.float32(1.0 / 6.0)  # scale 1: v = 6 x within row blocks
    for offset in (0, 5):
        qr, qc = gpu_quantize(dev_bf16(bits), ts, lib.SR, seed=seed, offset=offset)
        assert_quant_equal(qr, bits, ts, lib.SR, seed, offset, 0)
        assert_quant_equal(qc, bits, ts, lib.SR, seed, offset, 1)


def test_config3_gradient_sr_whole_tensor(cuda_device):
    """Stochastic rounding of config 3's whole 8192 x 4096 gradient, both
    orientations, every output row bit-exact with the oracle (67 M rounding
    decisions).  Rounding decisions whose fraction sits within 2^-22 above the
    random threshold are where the SR conversion instruction, which keeps 22
    bits of the fraction, would differ from the definition on its own (rows
    2455 of the row-wise output and 13, 3102, 3577 of the transposed one, with
    this seed); the kernels pre-round |v| up to a multiple of 2^-17 first."""
    d = config(3)
    dY = d["dY"]
    ts = fresh_ts(dY)
    qr, qc = gpu_quantize(dev_bf16(dY), ts, lib.SR, seed=sr_seed(3), offset=0)
    assert_quant_equal(qr, dY, ts, lib.SR, sr_seed(3), 0, 0)
    assert_quant_equal(qc, dY, ts, lib.SR, sr_seed(3), 0, 1)


def test_r4_operation_order_blocks(cuda_device):
    """The worked blocks that separate reading R4's order of roundings from
    its alternatives (tests/test_oracle_r4_order.py: tensor scales that are
    not powers of two, values within one fp32 ulp of a UE5M3 or E2M1
    midpoint), placed in row 0 and column 0 of a 16 x 16 tile so both output
    orientations see them: the kernels' codes and scales equal the oracle's,
    with round to nearest and with stochastic rounding."""
    from test_oracle_r4_order import ELEMENT_CASES, SCALE_CASES

    cases = [(a, t, 0) for a, t in SCALE_CASES] + [(a, t, x) for x, t, a in ELEMENT_CASES]
    for amax_b, ts_b, x_b in cases:
        tile = np.zeros((16, 16), dtype=np.uint16)
        tile[0, 0] = amax_b
        tile[0, 5] = tile[5, 0] = x_b
        tile[0, 9] = tile[9, 0] = 0x8000 | x_b  # and its negative
        ts = np.uint32(ts_b).view(np.float32)
        for rounding in (lib.RNE, lib.SR):
            qr, qc = gpu_quantize(dev_bf16(tile), ts, rounding, seed=5, offset=1)
            assert_quant_equal(qr, tile, ts, rounding, 5, 1, 0)
            assert_quant_equal(qc, tile, ts, rounding, 5, 1, 1)

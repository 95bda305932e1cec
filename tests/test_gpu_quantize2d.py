"""GPU parity of the 2-D (16 x 16 tile) quantizer with the oracle.

"Stable FP4 Training via Transposition-Invariant Block Quantization"
(summary in the UE5M3 paper's related-papers list): one scale per 16 x 16
tile, so the row-wise and the transposed operand hold the same codes.  Codes
and scale bytes must match the oracle (oracle/quantize2d.py) bit-exactly.
"""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import formats, quantize, quantize2d
from workloads import config, random_bf16, to_bf16_bits, STALE_FACTORS

from devhelpers import assert_gemm_close, dev_bf16, dev_scalar, fresh_ts, host

pytestmark = pytest.mark.gpu

MODES = [lib.RNE, lib.SR]


def gpu_quantize_2d(x_dev, ts, rounding, seed=0, offset=0, row=True, col=True, amax=None):
    rows, cols = x_dev.shape
    ts_dev = ts if hasattr(ts, "is_cuda") else dev_scalar(ts)
    qr = lib.empty_quantized(rows, cols, ts_dev) if row else None
    qc = lib.empty_quantized(cols, rows, ts_dev) if col else None
    lib.quantize_blockscale_2d(x_dev, ts_dev, rounding, seed, offset, row=qr, col=qc, amax=amax)
    return qr, qc


def assert_2d_equal(qr, qc, bits, ts, rounding, seed, offset, row0=0):
    """Bit-exact codes and scales against the oracle (rows row0 .. of the
    tensor when qr/qc were sliced to bits' rows)."""
    rc, rs, cc, cs, _ = quantize2d.quantize_blockscale_2d(bits, ts, rounding, seed, offset, row0)
    for name, got, want in (("row codes", qr and qr[0], rc), ("row scales", qr and qr[1], rs),
                            ("col codes", qc and qc[0], cc), ("col scales", qc and qc[1], cs)):
        if got is None:
            continue
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{name} mismatch at {bad[:5].tolist()}: gpu {got[tuple(bad[0])]:#x} "
                               f"oracle {want[tuple(bad[0])]:#x}")


def _host_pair(q):
    return None if q is None else (host(q.codes), host(q.scales))


@pytest.mark.parametrize("rounding", MODES)
@pytest.mark.parametrize("shape,kind", [((64, 256), "normal"), ((144, 544), "heavy"),
                                        ((400, 48), "gradient"), ((16, 16), "normal"),
                                        ((1024, 1040), "logrange"), ((336, 784), "heavy")])
def test_quantize2d_full_compare(cuda_device, rounding, shape, kind):
    """Whole outputs: several 64 x 256 workgroup tiles plus ragged edges."""
    bits = random_bf16(shape, seed=sum(shape) + 7, kind=kind)
    ts = fresh_ts(bits)
    amax = dev_scalar(0.0)
    qr, qc = gpu_quantize_2d(dev_bf16(bits), ts, rounding, seed=42, offset=5, amax=amax)
    assert_2d_equal(_host_pair(qr), _host_pair(qc), bits, ts, rounding, 42, 5)
    assert host(amax)[0] == quantize.tensor_amax(bits)
    # transposition invariance holds on the device output itself (a property
    # of the GPU's outputs, unpacked here without the oracle)
    def nibbles(packed):
        return np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[0], -1)

    assert np.array_equal(nibbles(host(qc.codes)), nibbles(host(qr.codes)).T)


def test_single_outputs_agree_with_fused(cuda_device):
    bits = random_bf16((192, 512), seed=13, kind="heavy")
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    for rounding in MODES:
        qr, qc = gpu_quantize_2d(x, ts, rounding, seed=5, offset=9)
        qr1, _ = gpu_quantize_2d(x, ts, rounding, seed=5, offset=9, col=False)
        _, qc1 = gpu_quantize_2d(x, ts, rounding, seed=5, offset=9, row=False)
        for a, b in ((qr.codes, qr1.codes), (qr.scales, qr1.scales), (qc.codes, qc1.codes),
                     (qc.scales, qc1.scales)):
            assert np.array_equal(host(a), host(b))


def test_strided_input(cuda_device):
    wide = random_bf16((128, 320), seed=43, kind="gradient")
    x = dev_bf16(wide)[:, 32:288]
    bits = np.ascontiguousarray(wide[:, 32:288])
    assert x.stride(0) == 320
    ts = fresh_ts(bits)
    qr, qc = gpu_quantize_2d(x, ts, lib.SR, seed=1, offset=2)
    assert_2d_equal(_host_pair(qr), _host_pair(qc), bits, ts, lib.SR, 1, 2)


def test_nonfinite_and_zero_tiles(cuda_device):
    bits = random_bf16((96, 272), seed=3, kind="normal")
    x = formats.bf16_to_f32(bits).copy()
    x[5, 7] = np.nan
    x[20, 100] = np.inf
    x[70, 260] = -np.inf
    x[32:48, 16:32] = 0.0
    x[48:64, 32:48] = -0.0
    bits = to_bf16_bits(x)
    for rounding in MODES:
        qr, qc = gpu_quantize_2d(dev_bf16(bits), 0.01, rounding, seed=8, offset=1)
        assert_2d_equal(_host_pair(qr), _host_pair(qc), bits, np.float32(0.01), rounding, 8, 1)
        sc = host(qr.scales)
        assert sc[5, 0] == 0xFF and sc[20, 6] == 0xFF and sc[70, 16] == 0xFF and sc[40, 1] == 0


@pytest.mark.parametrize("ts", [2.0 ** -120, 1e-30, 3.0e30, 2.0 ** 110])
def test_extreme_tensor_scales(cuda_device, ts):
    """Tensor scales outside the fast path's range take the general path."""
    bits = random_bf16((64, 96), seed=17, kind="logrange")
    for rounding in MODES:
        qr, qc = gpu_quantize_2d(dev_bf16(bits), ts, rounding, seed=2, offset=2)
        assert_2d_equal(_host_pair(qr), _host_pair(qc), bits, np.float32(ts), rounding, 2, 2)


@pytest.mark.parametrize("factor", STALE_FACTORS)
def test_stale_scale_log_range(cuda_device, factor):
    """The dynamic-range stress tensors (log-uniform block magnitudes) under
    a stale tensor scale: flushed and subnormal tile scales included."""
    cfg = config(5)
    bits = cfg["dY"][:512]
    ts = np.float32(np.float32(quantize.tensor_amax(bits) * np.float32(factor)) / np.float32(43008.0))
    for rounding in MODES:
        qr, qc = gpu_quantize_2d(dev_bf16(bits), ts, rounding, seed=11, offset=0)
        assert_2d_equal(_host_pair(qr), _host_pair(qc), bits, ts, rounding, 11, 0)


def test_full_size_sampled(cuda_device):
    """The activation-sized tensor (8192 x 4096, heavy-tailed with outlier
    columns) in the launch configuration the benchmark uses; sampled 16-row
    groups and column slices compared with the oracle."""
    cfg = config(2)
    bits = cfg["X"]
    ts = fresh_ts(bits)
    x = dev_bf16(bits)
    for rounding in MODES:
        qr, qc = gpu_quantize_2d(x, ts, rounding, seed=1002, offset=0, amax=dev_scalar(0.0))
        rc, rs, cc, cs = host(qr.codes), host(qr.scales), host(qc.codes), host(qc.scales)
        for g in (0, 1, 255, 256, 511):
            r0 = 16 * g
            o = quantize2d.quantize_blockscale_2d(bits[r0:r0 + 16], ts, rounding, 1002, 0, row0=r0)
            np.testing.assert_array_equal(rc[r0:r0 + 16], o[0])
            np.testing.assert_array_equal(rs[r0:r0 + 16], o[1])
            np.testing.assert_array_equal(cc[:, r0 // 2:r0 // 2 + 8], o[2])
            np.testing.assert_array_equal(cs[:, g:g + 1], o[3])


def test_2d_operands_feed_the_gemms(cuda_device):
    """One 2-D quantization of W serves fprop (row output) and dgrad (col
    output); both GEMMs match the oracle on the dequantized operands."""
    import torch

    X = random_bf16((256, 384), seed=71)
    W = random_bf16((320, 384), seed=72)
    dY = random_bf16((256, 320), seed=73, kind="gradient")
    tx, tw, tg = fresh_ts(X), fresh_ts(W), fresh_ts(dY)
    xr, _ = gpu_quantize_2d(dev_bf16(X), tx, lib.RNE, col=False)
    wr, wc = gpu_quantize_2d(dev_bf16(W), tw, lib.RNE)
    gr, _ = gpu_quantize_2d(dev_bf16(dY), tg, lib.SR, seed=4, offset=0, col=False)
    y = torch.empty((256, 320), dtype=torch.float32, device="cuda")
    dx = torch.empty((256, 384), dtype=torch.float32, device="cuda")
    lib.gemm_fprop(xr, wr, y)
    lib.gemm_dgrad(gr, wc, dx)
    # the oracle's own 2-D quantization of the same inputs; the GPU's equals it
    ox = quantize2d.quantize_blockscale_2d(X, tx, lib.RNE)
    ow = quantize2d.quantize_blockscale_2d(W, tw, lib.RNE)
    og = quantize2d.quantize_blockscale_2d(dY, tg, lib.SR, 4, 0)
    assert_2d_equal(_host_pair(xr), None, X, tx, lib.RNE, 0, 0)
    assert_2d_equal(_host_pair(wr), _host_pair(wc), W, tw, lib.RNE, 0, 0)
    assert_2d_equal(_host_pair(gr), None, dY, tg, lib.SR, 4, 0)
    assert_gemm_close(host(y), ox[0], ox[1], tx, ow[0], ow[1], tw)
    assert_gemm_close(host(dx), og[0], og[1], tg, ow[2], ow[3], tw)

"""GPU parity of the GEMM whose epilogue quantizes its bf16 output for the
next linear layer ("format-aware fusion" article in the UFP4 page's
similar-articles list: scale computation and packing fused with the GEMM).

The bf16 output must be bit-identical to the plain bf16-output GEMM's (same
accumulation), and the fused codes and scales bit-identical to the oracle's
block-16 quantization of that bf16 output (row-wise and transposed,
round-to-nearest and stochastic)."""

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from oracle import quantize

from devhelpers import dev_scalar, host

pytestmark = pytest.mark.gpu


def _operand(rng, rows, k, ts, lo=0x40, hi=0xB0):
    import torch

    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, k // 16), dtype=np.uint8)
    return lib.Quantized(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), dev_scalar(ts))


def _run(a, b, out_ts, rounding, seed, offset, row, col):
    import torch

    M, N = a.rows, b.rows
    ts = dev_scalar(out_ts)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amax = dev_scalar(0.0)
    qr = lib.empty_quantized(M, N, ts) if row else None
    qc = lib.empty_quantized(N, M, ts) if col else None
    lib.gemm_nt_bf16_quantized(a, b, y, ts, rounding, seed, offset, row=qr, col=qc, amax=amax)
    return y, amax, qr, qc


def _check(a, b, out_ts, rounding, seed, offset, row=True, col=True):
    import torch

    y, amax, qr, qc = _run(a, b, out_ts, rounding, seed, offset, row, col)
    y_ref = torch.empty_like(y)
    lib.gemm_nt_bf16(a, b, y_ref)
    ybits = host(y.view(torch.int16)).view(np.uint16)
    assert np.array_equal(ybits, host(y_ref.view(torch.int16)).view(np.uint16)), "bf16 output differs"
    ts = np.float32(out_ts)
    for q, o in ((qr, 0), (qc, 1)):
        if q is None:
            continue
        oc, os_ = quantize.quantize_blockscale(ybits, ts, rounding, seed, offset, o)
        gs, gc = host(q.scales), host(q.codes)
        bad = np.argwhere(gs != os_)
        assert bad.size == 0, f"orientation {o}: scale mismatch at {bad[:5].tolist()}"
        bad = np.argwhere(gc != oc)
        assert bad.size == 0, f"orientation {o}: code mismatch at {bad[:5].tolist()}"
    y32 = formats_bf16(ybits)
    assert np.array_equal(np.isnan(host(amax)), [np.isnan(y32).any()])
    if not np.isnan(y32).any():
        assert host(amax)[0] == np.float32(np.max(np.abs(y32)))


def formats_bf16(bits):
    from oracle import formats

    return formats.bf16_to_f32(bits)


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (320, 400, 128), (512, 768, 1024), (48, 1040, 96),
                                   (16, 16, 16), (272, 528, 4112)])
def test_fused_output_quantization(cuda_device, rounding, M, N, K):
    """Several output tiles, ragged edge tiles, aligned and unaligned K."""
    rng = np.random.default_rng(M + 3 * N + 5 * K + rounding)
    a = _operand(rng, M, K, 0.5)
    b = _operand(rng, N, K, 2.0e-3)
    out_ts = np.float32(4.0 / 43008.0)
    _check(a, b, out_ts, rounding, seed=1000 + M, offset=7)


def test_single_orientations_and_ragged_rows(cuda_device):
    """Row-wise output alone allows any M; transposed output alone any N."""
    rng = np.random.default_rng(11)
    a = _operand(rng, 300, 256, 0.25)
    b = _operand(rng, 272, 256, 1.0e-2)
    _check(a, b, 1e-4, lib.SR, 5, 1, row=True, col=False)
    a2 = _operand(rng, 288, 128, 0.25)
    b2 = _operand(rng, 250, 128, 1.0e-2)
    _check(a2, b2, 1e-4, lib.RNE, 5, 1, row=False, col=True)


@pytest.mark.parametrize("out_ts", [1e-30, 3.0e30, 2.0 ** -120])
def test_extreme_output_tensor_scales(cuda_device, out_ts):
    """Tensor scales outside the fast path's range (flushed, saturated and
    general-path blocks)."""
    rng = np.random.default_rng(23)
    a = _operand(rng, 64, 128, 1.0)
    b = _operand(rng, 48, 128, 1.0)
    for rounding in (lib.RNE, lib.SR):
        _check(a, b, out_ts, rounding, 3, 3)


def test_nan_block_in_output(cuda_device):
    """A NaN operand scale poisons an output row: its blocks get scale 0xFF."""
    import torch

    rng = np.random.default_rng(31)
    a = _operand(rng, 64, 64, 1.0)
    sc = host(a.scales).copy()
    sc[9, 1] = 0xFF
    a = lib.Quantized(a.codes, torch.from_numpy(sc).cuda(), a.ts)
    b = _operand(rng, 32, 64, 1.0)
    for rounding in (lib.RNE, lib.SR):
        _check(a, b, 1e-3, rounding, 2, 0)


def test_k_zero_output_is_zero(cuda_device):
    import torch

    a = lib.Quantized(torch.empty((32, 0), dtype=torch.uint8, device="cuda"),
                      torch.empty((32, 0), dtype=torch.uint8, device="cuda"), dev_scalar(1.0))
    b = lib.Quantized(torch.empty((48, 0), dtype=torch.uint8, device="cuda"),
                      torch.empty((48, 0), dtype=torch.uint8, device="cuda"), dev_scalar(1.0))
    y, amax, qr, qc = _run(a, b, 1.0, lib.RNE, 0, 0, True, True)
    assert not host(y.float()).any() and host(amax)[0] == 0.0
    assert not host(qr.codes).any() and not host(qr.scales).any()
    assert not host(qc.codes).any() and not host(qc.scales).any()

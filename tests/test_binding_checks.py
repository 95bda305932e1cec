"""CPU tests of the Python binding's argument checks: every malformed operand
is rejected with ValueError before a pointer is taken or anything launched.

The operands are stand-ins that claim to live on the GPU (`is_cuda`,
device cuda:0) but hold host tensors and fail if their address is ever
requested, so these tests need no GPU and prove that the check comes first.
A host tensor where the library expects device memory (a tensor scale left
on the CPU, say) is rejected the same way.
"""

import pytest
import torch

import fp4_block_scaled_amax_amd as lib

DEV = torch.device("cuda:0")


class Dev:
    """A host tensor presented as a device tensor; data_ptr() must not be called."""

    def __init__(self, t):
        self._t = t

    is_cuda = True
    device = DEV

    @property
    def dtype(self):
        return self._t.dtype

    @property
    def shape(self):
        return self._t.shape

    def dim(self):
        return self._t.dim()

    def numel(self):
        return self._t.numel()

    def is_contiguous(self):
        return self._t.is_contiguous()

    def stride(self, i):
        return self._t.stride(i)

    def data_ptr(self):  # pragma: no cover - reaching this is the failure
        raise AssertionError("a pointer was taken before the arguments were checked")

    def __getitem__(self, idx):
        return Dev(self._t[idx])

    def t(self):
        return Dev(self._t.t())


def u8(*shape):
    return Dev(torch.zeros(shape, dtype=torch.uint8))


def f32(*shape):
    return Dev(torch.zeros(shape, dtype=torch.float32))


def operand(rows, cols, ts=None):
    return lib.Quantized(u8(rows, cols // 2), u8(rows, cols // 16), ts if ts is not None else f32(1))


def raises(fn, match=None):
    with pytest.raises(ValueError, match=match):
        fn()


def test_gemm_rejects_host_tensor_scale():
    a, b = operand(32, 64), operand(48, 64)
    a.ts = torch.ones(1)  # left on the CPU: its host address must never reach a kernel
    raises(lambda: lib.gemm_nt(a, b, f32(32, 48)), "ts must be a device")


def test_gemm_rejects_host_codes_and_output():
    a, b = operand(32, 64), operand(48, 64)
    raises(lambda: lib.gemm_nt(lib.Quantized(torch.zeros((32, 32), dtype=torch.uint8), a.scales, a.ts), b,
                               f32(32, 48)), "device")
    raises(lambda: lib.gemm_nt(a, b, torch.zeros((32, 48))), "device")


@pytest.mark.parametrize("fn", ["gemm_nt", "gemm_fprop", "gemm_dgrad", "gemm_wgrad", "gemm_nt_bf16"])
def test_gemm_operand_checks(fn):
    call = getattr(lib, fn)
    out = (Dev(torch.zeros((32, 48), dtype=torch.bfloat16)) if fn == "gemm_nt_bf16" else f32(32, 48))
    good_a, good_b = operand(32, 64), operand(48, 64)
    bad = {
        "scales shape": lib.Quantized(u8(32, 32), u8(32, 3), f32(1)),
        "ts with 2 elements": lib.Quantized(u8(32, 32), u8(32, 4), f32(2)),
        "ts dtype": lib.Quantized(u8(32, 32), u8(32, 4), Dev(torch.zeros(1, dtype=torch.float64))),
        "strided codes": lib.Quantized(u8(32, 64)[:, ::2], u8(32, 4), f32(1)),
        "strided scales": lib.Quantized(u8(32, 32), u8(32, 8)[:, ::2], f32(1)),
        "codes dtype": lib.Quantized(Dev(torch.zeros((32, 32), dtype=torch.int16)), u8(32, 4), f32(1)),
        "cols not a multiple of 16": lib.Quantized(u8(32, 4), u8(32, 0), f32(1)),
        "not a Quantized": (u8(32, 32), u8(32, 4)),
    }
    for name, a in bad.items():
        with pytest.raises(ValueError):
            call(a, good_b, out)
        with pytest.raises(ValueError):
            call(good_a, a if name != "not a Quantized" else (u8(48, 32), u8(48, 4)), out)
    # K mismatch, wrong output shape, strided output
    raises(lambda: call(good_a, operand(48, 80), out))
    raises(lambda: call(good_a, good_b, f32(48, 32)))
    raises(lambda: call(good_a, good_b, f32(32, 96)[:, ::2]))


def test_quantize_output_checks():
    x = Dev(torch.zeros((64, 128), dtype=torch.int16))
    ts, amax = f32(1), f32(1)
    good_r, good_c = operand(64, 128), operand(128, 64)
    raises(lambda: lib.quantize_blockscale(x, ts, row=lib.Quantized(u8(64, 128)[:, ::2], u8(64, 8), ts)),
           "contiguous")
    raises(lambda: lib.quantize_blockscale(x, ts, row=lib.Quantized(u8(64, 64), u8(64, 7), ts)))
    raises(lambda: lib.quantize_blockscale(x, ts, col=lib.Quantized(u8(64, 64), u8(64, 8), ts)))
    raises(lambda: lib.quantize_blockscale(x, f32(3), row=good_r), "exactly one")
    raises(lambda: lib.quantize_blockscale(x, torch.ones(1), row=good_r), "device")
    raises(lambda: lib.quantize_blockscale(x, ts, row=good_r, amax=torch.zeros(1)), "device")
    raises(lambda: lib.quantize_blockscale_2d(x, ts, col=(u8(128, 32), u8(128, 3))))
    raises(lambda: lib.quantize_current_scaling(x, ts, f32(2), row=good_r), "exactly one")
    raises(lambda: lib.quantize_current_scaling(x, ts, amax, col=(u8(128, 32)[::2], u8(64, 4))))
    # x with a non-unit column stride
    raises(lambda: lib.quantize_blockscale(x.t(), ts, row=good_c), "unit stride")


def test_dequantize_update_and_mxfp4_checks():
    q = operand(16, 32)
    raises(lambda: lib.dequantize(q, f32(16, 64)[:, ::2]), "contiguous")
    raises(lambda: lib.dequantize(lib.Quantized(q.codes, q.scales, torch.ones(1)), f32(16, 32)), "device")
    raises(lambda: lib.update_tensor_scale(f32(1), f32(4), 0), "exactly one")
    raises(lambda: lib.update_tensor_scale(torch.zeros(1), f32(1), 0), "device")
    ac, asc = u8(32, 32), u8(32, 2)
    raises(lambda: lib.gemm_nt_mxfp4(ac, asc, torch.ones(1), u8(16, 32), u8(16, 2), f32(1), f32(32, 16)),
           "device")
    raises(lambda: lib.gemm_nt_mxfp4(u8(32, 64)[:, ::2], asc, f32(1), u8(16, 32), u8(16, 2), f32(1),
                                     f32(32, 16)), "contiguous")
    raises(lambda: lib.gemm_nt_mxfp4(ac, asc, f32(1), u8(16, 32), u8(16, 3), f32(1), f32(32, 16)))


def test_quantizing_epilogue_checks():
    a, b = operand(32, 64), operand(48, 64)
    out = Dev(torch.zeros((32, 48), dtype=torch.bfloat16))
    ts = f32(1)
    raises(lambda: lib.gemm_nt_bf16_quantized(a, b, out, torch.ones(1), row=operand(32, 48)), "device")
    raises(lambda: lib.gemm_nt_bf16_quantized(a, b, out, ts, row=operand(48, 32)))
    raises(lambda: lib.gemm_nt_bf16_quantized(a, b, out, ts, col=lib.Quantized(u8(48, 32)[:, ::2], u8(48, 2), ts)))


def test_stream_reference_checks():
    x = Dev(torch.zeros((32, 64), dtype=torch.bfloat16))
    good_r, good_c = (u8(32, 32), u8(32, 4)), (u8(64, 16), u8(64, 2))
    raises(lambda: lib.stream_reference(x, None), "row is required")
    raises(lambda: lib.stream_reference(Dev(torch.zeros((32, 40), dtype=torch.bfloat16)), good_r), "multiple of 16")
    raises(lambda: lib.stream_reference(torch.zeros((32, 64), dtype=torch.bfloat16), good_r), "device")
    raises(lambda: lib.stream_reference(x, (u8(32, 16), u8(32, 4))), "do not match")
    raises(lambda: lib.stream_reference(x, good_r, (u8(32, 32), u8(32, 4))), "do not match")
    raises(lambda: lib.stream_reference(x[:, ::2], good_r), "contiguous")

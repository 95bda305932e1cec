"""Every call launches on the stream it is given (the C ABI's `stream`
argument; the binding passes torch's current stream when none is given),
and calls from several host threads at once do not interfere.

A side stream first spins for a bounded time (torch.cuda._sleep) and then
copies the input into x.  A call on that stream is ordered after the copy;
a launch anywhere else would run during the spin and read x's old contents
(zeros), so the outputs would differ from the reference.  Buffers the calls
write are allocated and cleared on the side stream too.  The references come
from plain calls on the default stream after a full synchronization.
"""

from contextlib import nullcontext

import numpy as np
import pytest

import fp4_block_scaled_amax_amd as lib
from devhelpers import dev_bf16, dev_scalar, fresh_ts
from workloads import random_bf16

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000  # milliseconds at the GPU's clock


def _on(stream):
    import torch

    return torch.cuda.stream(stream) if stream is not None else nullcontext()


def _quantize(x, ts, rounding, stream=None):
    import torch

    R, C = x.shape
    with _on(stream):
        qr, qc = lib.empty_quantized(R, C, ts), lib.empty_quantized(C, R, ts)
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    lib.quantize_blockscale(x, ts, rounding, 7, 3, row=qr, col=qc, amax=amax, stream=stream)
    return qr, qc, amax


def _delayed_copy(stream, dst, src):
    import torch

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
        dst.copy_(src)


@pytest.fixture(scope="module")
def inputs(cuda_device):
    bits = random_bf16((2048, 4096), seed=77)
    return dev_bf16(bits), dev_scalar(fresh_ts(bits))


@pytest.mark.parametrize("rounding", [lib.RNE, lib.SR])
def test_quantize_runs_on_the_given_stream(inputs, rounding):
    import torch

    src, ts = inputs
    ref_r, ref_c, ref_a = _quantize(src, ts, rounding)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    x = torch.zeros_like(src)
    _delayed_copy(s, x, src)
    qr, qc, amax = _quantize(x, ts, rounding, stream=s)  # the current stream is the default one here
    s.synchronize()
    for a, b in ((qr.codes, ref_r.codes), (qr.scales, ref_r.scales), (qc.codes, ref_c.codes),
                 (qc.scales, ref_c.scales), (amax, ref_a)):
        assert bool(torch.equal(a, b))


def test_a_launch_on_another_stream_would_be_caught(inputs):
    """Control: the same call issued on the default stream while the side
    stream spins reads x before the copy (all zeros), so its outputs differ
    from the reference -- the set-up above detects a launch on the wrong
    stream."""
    import torch

    src, ts = inputs
    ref_r, _, _ = _quantize(src, ts, lib.RNE)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    x = torch.zeros_like(src)
    _delayed_copy(s, x, src)
    qr, _, amax = _quantize(x, ts, lib.RNE, stream=torch.cuda.default_stream())
    torch.cuda.default_stream().synchronize()
    early = (qr.codes.clone(), qr.scales.clone(), amax.clone())
    s.synchronize()
    assert not bool(torch.equal(early[0], ref_r.codes))
    assert int(early[1].count_nonzero()) == 0 and float(early[2]) == 0.0  # it saw the zeros


def test_current_stream_is_the_default(inputs):
    import torch

    src, ts = inputs
    ref_r, ref_c, _ = _quantize(src, ts, lib.RNE)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    x = torch.zeros_like(src)
    _delayed_copy(s, x, src)
    with torch.cuda.stream(s):
        qr, qc, _ = _quantize(x, ts, lib.RNE)  # no stream argument: torch's current stream, s
    s.synchronize()
    assert bool(torch.equal(qr.codes, ref_r.codes)) and bool(torch.equal(qc.scales, ref_c.scales))


def test_refresh_and_gemms_run_on_the_given_stream(inputs):
    """The amax pass, the tensor-scale refresh, the quantization and the
    three GEMM entry points chained on a side stream behind the delayed copy
    (shapes from X alone: Y = X X^T, dX = X X^T, dW = X^T X)."""
    import torch

    src, _ = inputs
    R, C = src.shape

    def chain(x, stream):
        with _on(stream):
            amax = torch.zeros(1, dtype=torch.float32, device="cuda")
            ts = torch.ones(1, dtype=torch.float32, device="cuda")
            qr, qc = lib.empty_quantized(R, C, ts), lib.empty_quantized(C, R, ts)
            y = torch.empty((R, R), dtype=torch.float32, device="cuda")
            dx = torch.empty((R, R), dtype=torch.float32, device="cuda")
            dw = torch.empty((C, C), dtype=torch.float32, device="cuda")
        lib.quantize_blockscale(x, None, amax=amax, stream=stream)
        lib.update_tensor_scale(amax, ts, 0, 1, stream=stream)
        lib.quantize_blockscale(x, ts, lib.RNE, row=qr, col=qc, stream=stream)
        lib.gemm_fprop(qr, qr, y, stream=stream)   # tokens R, in C, out R
        lib.gemm_dgrad(qr, qr, dx, stream=stream)  # dY: R x C (out C); W^T operand: R x C (in R)
        lib.gemm_wgrad(qc, qc, dw, stream=stream)  # dY^T: C x R (out C); X^T: C x R (in C)
        return ts, qr.codes, qc.scales, y, dx, dw

    ref = chain(src, None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    x = torch.zeros_like(src)
    _delayed_copy(s, x, src)
    got = chain(x, s)
    s.synchronize()
    for i, (a, b) in enumerate(zip(got, ref)):
        assert bool(torch.equal(a, b)), f"output {i} differs"
    assert float(np.abs(got[3].cpu().numpy()).max()) > 0.0


def test_concurrent_calls_from_two_host_threads(inputs):
    """The library keeps no state: two host threads (ctypes releases the
    interpreter lock during each call) quantizing and running fprop on their
    own streams at the same time get the results of serial calls."""
    import threading

    import torch

    src, ts = inputs
    R, C = src.shape
    ref_r, ref_c, ref_a = _quantize(src, ts, lib.SR)
    y_ref = torch.empty((R, R), dtype=torch.float32, device="cuda")
    lib.gemm_fprop(ref_r, ref_r, y_ref)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(tid):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(20):
                    qr, qc, amax = _quantize(src, ts, lib.SR)
                    y = torch.empty((R, R), dtype=torch.float32, device="cuda")
                    lib.gemm_fprop(qr, qr, y)
                    s.synchronize()
                    ok = (torch.equal(qr.codes, ref_r.codes) and torch.equal(qc.scales, ref_c.scales)
                          and torch.equal(amax, ref_a) and torch.equal(y, y_ref))
                    results[(tid, it)] = bool(ok)
        except Exception as ex:  # reported below
            errors.append(repr(ex))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not errors, errors
    assert len(results) == 40 and all(results.values())

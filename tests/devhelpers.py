"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI (via the binding), and compare with the oracle."""

import numpy as np

import fp4_block_scaled_amax_amd as lib
from oracle import gemm, quantize, tensor_scale


def dev_bf16(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def dev_scalar(v):
    import torch

    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda")


def fresh_ts(bits):
    """Tensor scale refreshed from this tensor's own amax (oracle arithmetic)."""
    _, ts = tensor_scale.update_tensor_scale(quantize.tensor_amax(bits), np.float32(1.0), 0, 1)
    return ts


def gpu_quantize(x_dev, ts, rounding=lib.RNE, seed=0, offset=0, row=True, col=True, amax=None):
    """Returns (row Quantized or None, col Quantized or None)."""
    rows, cols = x_dev.shape
    ts_dev = ts if hasattr(ts, "is_cuda") else dev_scalar(ts)
    qr = lib.empty_quantized(rows, cols, ts_dev) if row else None
    qc = lib.empty_quantized(cols, rows, ts_dev) if col else None
    lib.quantize_blockscale(x_dev, ts_dev, rounding, seed, offset, row=qr, col=qc, amax=amax)
    return qr, qc


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_quant_equal(q_dev, bits, ts, rounding, seed, offset, orientation, rows=None):
    """Bit-exact comparison of codes and scales with the oracle, on all output
    rows or on the sampled output rows `rows`."""
    codes = host(q_dev.codes)
    scales = host(q_dev.scales)
    oc, os_ = quantize.quantize_blockscale(bits, ts, rounding, seed, offset, orientation, rows=rows)
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    bad_s = np.argwhere(scales != os_)
    assert bad_s.size == 0, f"scale mismatch at {bad_s[:5].tolist()}: gpu {scales[tuple(bad_s[0])]:#x} oracle {os_[tuple(bad_s[0])]:#x}"
    bad_c = np.argwhere(codes != oc)
    assert bad_c.size == 0, f"code mismatch at {bad_c[:5].tolist()}: gpu {codes[tuple(bad_c[0])]:#x} oracle {oc[tuple(bad_c[0])]:#x}"


def assert_gemm_close(c_gpu, a_codes, a_scales, ts_a, b_codes, b_scales, ts_b, rows=None, cols=None,
                      rtol=1e-5):
    """|C_gpu - C_ref| <= rtol * |tsA tsB| * sum|a||b| per element, on all
    elements or on the sampled (rows[t], cols[t]) entries.  NaN must match.
    The operands are the oracle's (never codes the GPU produced)."""
    if rows is None:
        ref, bound = gemm.gemm_nt(a_codes, a_scales, ts_a, b_codes, b_scales, ts_b)
        got = c_gpu.astype(np.float64)
        return _close(got, ref, bound, rtol)
    return assert_entries_close(c_gpu[rows, cols], a_codes, a_scales, ts_a, b_codes, b_scales, ts_b,
                                rows, cols, rtol)


def assert_entries_close(got, a_codes, a_scales, ts_a, b_codes, b_scales, ts_b, ia, ib, rtol=1e-5):
    """GPU entries got[t] against entry (ia[t], ib[t]) of the oracle's
    tsA tsB A B^T, where A and B hold only the operand rows the entries use."""
    ref, bound = gemm.gemm_nt_entries(a_codes, a_scales, ts_a, b_codes, b_scales, ts_b, ia, ib)
    return _close(np.asarray(got).astype(np.float64), ref, bound, rtol)


def _close(got, ref, bound, rtol):
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "NaN pattern differs"
    err = np.abs(got - ref)[~nan_ref]
    lim = (rtol * bound)[~nan_ref]
    worst = np.argmax(err - lim) if err.size else 0
    assert np.all(err <= lim), (f"gemm error {err.flat[worst]:.3e} > {lim.flat[worst]:.3e} "
                                f"(ref {ref[~nan_ref].flat[worst]:.6e})")
    return float(np.max(err / np.maximum(bound[~nan_ref], 1e-300))) if err.size else 0.0


def oracle_operand(bits, ts, rounding, seed, offset, orientation, q_gpu=None, rows=None):
    """The oracle's quantization of bf16 `bits` in one orientation (output
    rows `rows` only, with their true coordinates, when given).  With q_gpu,
    the GPU's codes and scales on those rows must equal it bit for bit.
    Returns (codes, scales)."""
    codes, scales = quantize.quantize_blockscale(bits, ts, rounding, seed, offset, orientation, rows=rows)
    if q_gpu is not None:
        gc, gs = host(q_gpu.codes), host(q_gpu.scales)
        if rows is not None:
            gc, gs = gc[rows], gs[rows]
        assert np.array_equal(gs, scales), f"scales differ (orientation {orientation})"
        assert np.array_equal(gc, codes), f"codes differ (orientation {orientation})"
    return codes, scales


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(k, n), replace=False)
    pick[:2] = [0, n - 1] if n > 1 else [0, 0]
    return np.unique(pick)

"""The library under HIP graph capture: a slice of a training step -- the
quantizers (1-D, 2-D, current scaling, amax by-product), the three GEMMs,
the quantizing epilogue and the tensor-scale refresh -- captured once in a
graph and replayed several times, with eager work and synchronizations
between the replays.  Every replay must reproduce the eager step bit for bit
(no call records a memset node: scalars are cleared by kernels)."""

import pytest

import fp4_block_scaled_amax_amd as lib
from workloads import random_bf16

from devhelpers import dev_bf16, dev_scalar, fresh_ts

pytestmark = pytest.mark.gpu


def test_step_slice_graph_replays_match_eager(cuda_device):
    import torch

    T, I, O = 512, 256, 384
    X = dev_bf16(random_bf16((T, I), 1))
    W = dev_bf16(random_bf16((O, I), 2))
    G = dev_bf16(random_bf16((T, O), 3, "gradient"))
    state = {
        "ts_x": dev_scalar(fresh_ts(random_bf16((T, I), 1))), "ts_w": dev_scalar(fresh_ts(random_bf16((O, I), 2))),
        "ts_g": dev_scalar(fresh_ts(random_bf16((T, O), 3, "gradient"))), "ts_y": dev_scalar(1e-3),
        "ts_cur": dev_scalar(1.0), "amax_x": dev_scalar(0.0), "amax_w": dev_scalar(0.0),
        "amax_g": dev_scalar(0.0), "amax_y": dev_scalar(0.0), "amax_cur": dev_scalar(0.0),
    }
    q = {
        "xr": lib.empty_quantized(T, I, state["ts_x"]), "xc": lib.empty_quantized(I, T, state["ts_x"]),
        "wr": lib.empty_quantized(O, I, state["ts_w"]), "wc": lib.empty_quantized(I, O, state["ts_w"]),
        "gr": lib.empty_quantized(T, O, state["ts_g"]), "gc": lib.empty_quantized(O, T, state["ts_g"]),
        "yr": lib.empty_quantized(T, O, state["ts_y"]), "yc": lib.empty_quantized(O, T, state["ts_y"]),
        "cr": lib.empty_quantized(T, I, state["ts_cur"]),
        "x2r": lib.empty_quantized(T, I, state["ts_x"]), "x2c": lib.empty_quantized(I, T, state["ts_x"]),
    }
    out = {
        "y": torch.empty((T, O), dtype=torch.float32, device="cuda"),
        "dx": torch.empty((T, I), dtype=torch.float32, device="cuda"),
        "dw": torch.empty((O, I), dtype=torch.float32, device="cuda"),
        "y16": torch.empty((T, O), dtype=torch.bfloat16, device="cuda"),
    }

    def step():
        s = state
        lib.quantize_blockscale(X, s["ts_x"], lib.RNE, row=q["xr"], col=q["xc"], amax=s["amax_x"])
        lib.quantize_blockscale(W, s["ts_w"], lib.RNE, row=q["wr"], col=q["wc"], amax=s["amax_w"])
        lib.quantize_blockscale(G, s["ts_g"], lib.SR, 11, 3, row=q["gr"], col=q["gc"], amax=s["amax_g"])
        lib.gemm_fprop(q["xr"], q["wr"], out["y"])
        lib.gemm_dgrad(q["gr"], q["wc"], out["dx"])
        lib.gemm_wgrad(q["gc"], q["xc"], out["dw"])
        lib.gemm_nt_bf16_quantized(q["xr"], q["wr"], out["y16"], s["ts_y"], lib.RNE, row=q["yr"], col=q["yc"],
                                   amax=s["amax_y"])
        lib.quantize_current_scaling(X, s["ts_cur"], s["amax_cur"], lib.RNE, row=q["cr"])
        lib.quantize_blockscale_2d(X, s["ts_x"], lib.RNE, row=q["x2r"], col=q["x2c"])
        for a, t in (("amax_x", "ts_x"), ("amax_w", "ts_w"), ("amax_g", "ts_g"), ("amax_y", "ts_y")):
            lib.update_tensor_scale(s[a], s[t], 0, 1)

    def snapshot():
        snap = {k: v.clone() for k, v in state.items()}
        for k, v in q.items():
            snap[k + ".codes"], snap[k + ".scales"] = v.codes.clone(), v.scales.clone()
        for k, v in out.items():
            snap[k] = v.clone()
        return snap

    def restore(snap):
        for k, v in state.items():
            v.copy_(snap[k])

    initial = snapshot()
    step()  # eager reference (also loads the library's kernels before capture)
    torch.cuda.synchronize()
    eager = snapshot()

    restore(initial)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        restore(initial)
        for v in list(q.values()):
            v.codes.fill_(0x5A)
            v.scales.fill_(0x5A)
        for v in out.values():
            v.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in eager:
            assert torch.equal(got[k], eager[k]), f"replay {replay}: {k} differs from the eager step"
        # eager work between the replays
        torch.randn(1024, 1024, device="cuda").sum().item()

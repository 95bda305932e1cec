"""Benchmark of the UE5M3-FP4 hot path on one MI355X.

One step = the whole data-parallel hot path of an FFN pair's training step at
8192 tokens (hidden 4096, FFN 16384): for the up and the down projection,
quantize X and W (round-to-nearest) and dY (stochastic rounding) in both
orientations with the tensor-amax by-product, run fprop / dgrad / wgrad
(six 8192 x 4096 x 16384 block-scaled GEMMs in all), then refresh the six
tensor scales.  Inputs are seeded synthetic bf16 tensors resident in HBM
before timing starts.

Prints one JSON line.  `value` is the step's GEMM work (6 x 1.0995e12 flop)
divided by the measured step time, in TFLOP/s.  `roofline` is for the GEMM
kernel (the dominant kernel): algorithmic flops per launch over its average
launch time, measured with HIP events on the stream it runs on, against the
fp16 dense MFMA peak (the kernel feeds exact fp16 dequantizations to fp16
MFMA; fp16 and bf16 share the 2.5 PFLOP/s dense peak).  Its `traffic` is the
HBM bytes per launch from the committed rocprofv3 counter summary of this
command, reported only while the GEMM source still matches the one profiled.
`quantize` reports the quantizer's GB/s inside the step (round-to-nearest
and stochastic calls separately) and, as `quantize_activations`, on its own
over the 8192 x 4096 heavy-tailed activation workload with 8 rotating
HBM-resident buffer sets (the quantizer's bandwidth roofline).  Both carry
`frac_of_stream_reference`: the time of a kernel that moves the same bytes as
contiguous streams with no quantization, over the quantizer's time -- the
share of the HBM rate the quantizer's read/write mix can reach that it
reaches.
`epilogue_fusion` times the largest fprop of the step with its output fused
for the next layer (bf16 Y and its amax) against the fp32 output.
`native_mxfp4` times the native MXFP4 comparison GEMM at the step's GEMM
shape: its ratio to the UE5M3 GEMM is the cost of emulating UE5M3 scales.
`configs` reports the other workloads call by call: the tiny linear's
latency, eager and as HIP graph replays, next to the oracle's seconds
(256 x 256), the attention-projection
layer (8192 x 4096 x 4096) and the dynamic-range stress layer at 4096^3 with
stale tensor scales -- each quantization in GB/s, each GEMM in TFLOP/s.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step
(about 10-20 s of host work), with the threads it ran on, the host's CPU
count and the affinity mask.

`--copy-calibration` instead runs a plain 256 MiB device copy, whose
FETCH_SIZE / WRITE_SIZE counter readings give the scale factors that turn
those counters into bytes.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "UE5M3-FP4 GEMM TFLOP/s (fprop/dgrad/wgrad) + quantize GB/s, % roofline"
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 MFMA, MI355X
TOKENS, HIDDEN, FFN = 8192, 4096, 16384
QUANT_BYTES_PER_ELEM = 2.0 + 2 * 0.5625  # bf16 in; codes + scales out, both orientations
CPU_GEMM_ROWS = 4096  # output rows of the up projection's fprop in the oracle's timed sample
CPU_QUANT_ROWS = 3072  # output rows per orientation of dY_up in the oracle's timed sample


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1, help="GPUs to run on (one GPU only; more exits with a message)")
    p.add_argument("--steps", type=int, default=10, help="timed FFN-pair training steps")
    p.add_argument("--warmup", type=int, default=3, help="untimed steps before the timed ones")
    p.add_argument("--period", type=int, default=1, help="tensor-scale refresh period")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-quantize-only", action="store_true",
                   help="skip the stand-alone quantizer measurement")
    p.add_argument("--no-graph", action="store_true",
                   help="skip timing the step captured as one HIP graph")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the epilogue-fusion and native-MXFP4 comparisons")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-call figures of configs 1, 3 and 5")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a 256 MiB device copy (counter calibration)")
    return p.parse_args()


PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "gemm_nt_kernel_ffn_pair_counters.json")


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when the GEMM kernel (its source or its compile options) changed since
    the counters were taken."""
    from fp4_block_scaled_amax_amd.build import kernel_fingerprint

    try:
        with open(PROFILE_COUNTERS) as f:
            prof = json.load(f)
        digest = kernel_fingerprint("gemm.hip")
    except (OSError, ValueError):
        return None
    if prof.get("gemm_kernel_fingerprint") != digest:
        return None
    return float(prof["hbm_bytes_per_launch"])


def copy_calibration():
    import torch

    n = 256 * 1024 * 1024 // 4  # 256 MiB of fp32
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


class Tensor:
    """One bf16 operand of the step with its quantized buffers and scale state."""

    def __init__(self, lib, torch, bits, rounding, tid):
        self.x = torch.from_numpy(bits.view("int16")).cuda()
        rows, cols = bits.shape
        self.ts = torch.ones(1, dtype=torch.float32, device="cuda")
        self.amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.row = lib.empty_quantized(rows, cols, self.ts)
        self.col = lib.empty_quantized(cols, rows, self.ts)
        self.rounding = rounding
        self.tid = tid
        self.elems = rows * cols


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import fp4_block_scaled_amax_amd as lib
    from workloads import config, sr_seed

    lib.load_library()
    torch.cuda.set_device(0)
    data = config(4)
    cpu_sample = None
    if not args.no_cpu_baseline:  # the oracle's sample rows, kept before the device copies
        cpu_sample = {k: data[k] for k in ("dY_up", "W_up")}
        cpu_sample["X_rows"] = data["X"][:CPU_GEMM_ROWS].copy()
    seed = sr_seed(4)
    layers = []
    tid = 0
    for xn, wn, dn in (("X", "W_up", "dY_up"), ("H", "W_down", "dY_down")):
        X = Tensor(lib, torch, data[xn], lib.RNE, tid)
        W = Tensor(lib, torch, data[wn], lib.RNE, tid + 1)
        D = Tensor(lib, torch, data[dn], lib.SR, tid + 2)
        tid += 3
        tokens, in_f = data[xn].shape
        out_f = data[wn].shape[0]
        Y = torch.empty((tokens, out_f), dtype=torch.float32, device="cuda")
        dX = torch.empty((tokens, in_f), dtype=torch.float32, device="cuda")
        dW = torch.empty((out_f, in_f), dtype=torch.float32, device="cuda")
        layers.append((X, W, D, Y, dX, dW, tokens, in_f, out_f))
    del data
    tensors = [t for L in layers for t in L[:3]]
    n_tensors = len(tensors)
    gemm_flops = [2.0 * L[6] * L[7] * L[8] for L in layers for _ in range(3)]
    step_flops = float(sum(gemm_flops))
    quant_bytes = sum(t.elems for t in tensors) * QUANT_BYTES_PER_ELEM

    # bootstrap: amax-only pass, then the first refresh (step 0)
    for t in tensors:
        lib.quantize_blockscale(t.x, None, amax=t.amax)
        lib.update_tensor_scale(t.amax, t.ts, 0, 1)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(s, timing=None):
        for L in layers:
            X, W, D, Y, dX, dW = L[:6]
            for t in (X, W, D):
                e0 = ev() if timing is not None else None
                if e0:
                    e0.record()
                lib.quantize_blockscale(t.x, t.ts, t.rounding, seed, s * n_tensors + t.tid,
                                        row=t.row, col=t.col, amax=t.amax)
                if e0:
                    e1 = ev()
                    e1.record()
                    timing["quantize"].append((e0, e1, t.elems, t.rounding))
            for fn, a, b, c in ((lib.gemm_fprop, X.row, W.row, Y), (lib.gemm_dgrad, D.row, W.col, dX),
                                (lib.gemm_wgrad, D.col, X.col, dW)):
                e0 = ev() if timing is not None else None
                if e0:
                    e0.record()
                fn(a, b, c)
                if e0:
                    e1 = ev()
                    e1.record()
                    timing["gemm"].append((e0, e1, 2.0 * c.shape[0] * c.shape[1] * a.cols))
        for t in tensors:
            lib.update_tensor_scale(t.amax, t.ts, s + 1, args.period)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # timed region: K whole steps, wall clock and stream events
    timing = {"quantize": [], "gemm": []}
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.warmup, args.warmup + args.steps):
        step(s, timing)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps
    wall_ms = wall * 1e3 / args.steps

    gemm_ms = [a.elapsed_time(b) for a, b, _ in timing["gemm"]]
    gemm_fl = [f for _, _, f in timing["gemm"]]
    gemm_avg_ms = float(np.mean(gemm_ms))
    gemm_tflops = float(np.sum(gemm_fl) / (np.sum(gemm_ms) * 1e-3) / 1e12)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    def q_stats(rounding):
        sel = [(a.elapsed_time(b), n) for a, b, n, rnd in timing["quantize"] if rnd == rounding]
        ms = float(sum(m for m, _ in sel))
        gbs = sum(n for _, n in sel) * QUANT_BYTES_PER_ELEM / (ms * 1e-3) / 1e9
        return {"achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                "avg_launch_ms": round(ms / len(sel), 4), "launches_per_step": len(sel) // args.steps}

    # the streaming reference (same bytes, contiguous streams, no arithmetic)
    # on the step's six tensors in the step's order: the HBM rate each
    # rounding's quantize calls could reach with their read/write mix
    ref_ms = {lib.RNE: [], lib.SR: []}
    for p in range(4):
        evs = []
        for t in tensors:
            e0, e1 = ev(), ev()
            e0.record()
            lib.stream_reference(t.x, t.row, t.col)
            e1.record()
            evs.append((e0, e1, t.rounding))
        torch.cuda.synchronize()
        if p > 0:  # the first pass is a warm-up
            for e0, e1, rnd in evs:
                ref_ms[rnd].append(e0.elapsed_time(e1))

    def with_reference(stats, rounding):
        ref = float(np.mean(ref_ms[rounding]))
        stats["stream_reference_avg_launch_ms"] = round(ref, 4)
        stats["frac_of_stream_reference"] = round(ref / stats["avg_launch_ms"], 4)
        # what bounds it (rocprofv3 counters of these launches): round to
        # nearest streams HBM; stochastic rounding keeps the vector ALU busy
        # about 90 % of cycles (Philox and the SR conversion)
        stats["bound"] = "alu" if rounding == lib.SR else "hbm"
        return stats

    traffic = gemm_traffic()

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "ffn_pair_fwd_bwd", "tokens": TOKENS, "hidden": HIDDEN,
                   "ffn": FFN, "gemms_per_step": 6, "quantize_calls_per_step": 6,
                   "tensor_scale_period": args.period,
                   "gemm_shape": "8192x4096x16384 (M,N,K permuted)",
                   "formats": "E2M1 payload, UE5M3 block-16 scales, fp32 tensor scale; "
                              "GEMM: exact fp16 dequant (q*s/16) -> fp16 MFMA, fp32 accumulate; "
                              "quantizer arithmetic fp32"},
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": {"bound": "mfma", "kernel": "gemm_nt_kernel",
                     "achieved": round(gemm_tflops, 2), "peak": FP16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                     "avg_launch_ms": round(gemm_avg_ms, 4),
                     "flop_per_launch": gemm_fl[0],
                     "traffic": None if traffic is None else round(traffic)},
        "quantize": {"peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_elem": QUANT_BYTES_PER_ELEM,
                     "rne": with_reference(q_stats(lib.RNE), lib.RNE),
                     "sr": with_reference(q_stats(lib.SR), lib.SR)},
    }
    step_elems = sum(t.elems for t in tensors)
    if not args.no_graph:
        result["graph"] = graph_replay(torch, step, args, step_flops)
    if not args.no_extras:
        result["epilogue_fusion"] = epilogue_fusion(lib, torch, layers[0])
        result["native_mxfp4"] = native_mxfp4(lib, torch, gemm_tflops)
        result["dynamic_range_stress"] = dynamic_range_stress(lib, torch)
    del layers, tensors
    torch.cuda.empty_cache()
    if not args.no_quantize_only:
        result["quantize_activations"] = quantize_only(lib, torch)
    if not args.no_configs:
        result["configs"] = {"config1_tiny_linear": config1_latency(lib, torch),
                             "config3_attention_projection": linear_layer_timing(lib, torch, 3),
                             "config5_dynamic_range_stale_x8": linear_layer_timing(lib, torch, 5, stale=8.0)}
    if cpu_sample is not None:
        result["cpu_baseline"] = cpu_baseline(step_flops, step_elems, cpu_sample)
    print(json.dumps(result), flush=True)


def graph_replay(torch, step, args, step_flops):
    """The same step captured once as a HIP graph (torch.cuda.graph) and
    replayed `steps` times: what the step costs without per-launch host work.
    The captured step keeps one step's stochastic-rounding offsets and refresh
    decision; its outputs equal the eager step's (tests/test_gpu_graph.py)."""
    try:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step(args.warmup + args.steps)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        del g
        return {"ms_per_step": round(ms, 4), "value": round(step_flops / (ms * 1e-3) / 1e12, 2)}
    except Exception as ex:  # capture unsupported by this runtime: report, do not fail the run
        return f"unavailable: {type(ex).__name__}: {ex}"[:200]


def epilogue_fusion(lib, torch, up):
    """The up projection's fprop (8192 x 16384 x 4096, the largest output of
    the step) with its output fused for the next layer -- bf16 Y plus its
    tensor amax, and optionally Y's block-16 quantization (row-wise and
    transposed, round to nearest) in the epilogue -- against the fp32 output
    and against the bf16 output followed by the stand-alone quantizer, on the
    same quantized operands."""
    X, W = up[0], up[1]
    tokens, out_f = X.row.rows, W.row.rows
    y32 = torch.empty((tokens, out_f), dtype=torch.float32, device="cuda")
    y16 = torch.empty((tokens, out_f), dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    flop = 2.0 * tokens * out_f * X.row.cols
    res = {"shape": f"{tokens}x{out_f}x{X.row.cols}"}
    # the next linear's input quantization (block-16, both orientations,
    # round to nearest) fused into the epilogue, and done after it
    ts_y = torch.full((1,), 1.0 / 43008.0, dtype=torch.float32, device="cuda")
    qr = lib.empty_quantized(tokens, out_f, ts_y)
    qc = lib.empty_quantized(out_f, tokens, ts_y)
    for name, fn in (("fp32_out", lambda: lib.gemm_fprop(X.row, W.row, y32)),
                     ("bf16_out_amax", lambda: lib.gemm_nt_bf16(X.row, W.row, y16, amax=amax)),
                     ("bf16_out_amax_quantized_in_epilogue",
                      lambda: lib.gemm_nt_bf16_quantized(X.row, W.row, y16, ts_y, lib.RNE, row=qr, col=qc,
                                                         amax=amax)),
                     ("bf16_out_amax_then_quantize",
                      lambda: (lib.gemm_nt_bf16(X.row, W.row, y16, amax=amax),
                               lib.quantize_blockscale(y16, ts_y, lib.RNE, row=qr, col=qc)))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        res[name] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                     "output_bytes": tokens * out_f * (4 if name == "fp32_out" else 2)}
    del qr, qc
    return res


def native_mxfp4(lib, torch, ue5m3_tflops):
    """The cost of emulating UE5M3: the native MXFP4 comparison GEMM (E2M1 +
    E8M0 per 32 on the scaled FP4 MFMA, same tiling) at 8192 x 4096 x 16384
    on random operands, against the UE5M3 GEMM's average in the step; and,
    when this torch build provides it, the vendor library's MXFP4 GEMM (bf16
    output) with the same ratio to the UE5M3 GEMM."""
    M, N, K = TOKENS, HIDDEN, FFN
    g = torch.Generator(device="cuda").manual_seed(17)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    bc = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    asc = torch.randint(110, 140, (M, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    bsc = torch.randint(110, 140, (N, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    one = torch.ones(1, device="cuda")
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    flop = 2.0 * M * N * K

    def timed(fn, iters=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms = timed(lambda: lib.gemm_nt_mxfp4(ac, asc, one, bc, bsc, one, c))
    tf = flop / (ms * 1e-3) / 1e12
    res = {"shape": f"{M}x{N}x{K}", "ms": round(ms, 4), "tflops": round(tf, 1),
           "peak_fp4": 10100.0, "frac": round(tf / 10100.0, 4),
           "emulation_tax": round(tf / ue5m3_tflops, 3)}
    try:  # vendor comparison point, if supported by this torch build
        a4 = ac.view(torch.float4_e2m1fn_x2)
        b4 = bc.view(torch.float4_e2m1fn_x2)
        ms_v = timed(lambda: torch._scaled_mm(a4, b4.t(), scale_a=asc.view(torch.float8_e8m0fnu),
                                              scale_b=bsc.view(torch.float8_e8m0fnu),
                                              out_dtype=torch.bfloat16))
        tf_v = flop / (ms_v * 1e-3) / 1e12
        res["vendor_mxfp4_bf16_out"] = {"ms": round(ms_v, 4), "tflops": round(tf_v, 1),
                                        "emulation_tax": round(tf_v / ue5m3_tflops, 3)}
    except Exception as ex:  # pragma: no cover
        res["vendor_mxfp4_bf16_out"] = f"unavailable: {type(ex).__name__}"
    return res


def dynamic_range_stress(lib, torch):
    """The dynamic-range stress tensors (4096 x 4096, magnitudes log-uniform
    over 2^-24..2^12 per row block) quantized row-wise under a fresh tensor
    scale and under scales from an amax off by x8 and x1/8 (a stale periodic
    scale): fraction of blocks flushed to scale 0 although non-zero, of
    blocks with a subnormal UE5M3 scale, of saturated (0xFE) blocks, the
    relative L2 error of the dequantized tensor (which its largest blocks
    dominate), and the mean and median over non-zero blocks of each block's
    own relative L2 error (1 for a flushed block).  X with round to nearest,
    dY with stochastic rounding."""
    from workloads import STALE_FACTORS, config, sr_seed

    data = config(5)
    res = {"workload": "4096x4096, log-uniform block magnitudes 2^-24..2^12"}
    for name, rnd in (("X", lib.RNE), ("dY", lib.SR)):
        x = torch.from_numpy(data[name].view("int16")).cuda()
        xf = x.view(torch.bfloat16).float()
        R, C = xf.shape
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        lib.quantize_blockscale(x, None, amax=amax)
        blk_nonzero = xf.abs().view(R, C // 16, 16).amax(dim=2) > 0
        out = torch.empty((R, C), dtype=torch.float32, device="cuda")
        entry = {}
        for label, factor in [("fresh", 1.0)] + [(f"stale_x{f:g}", f) for f in STALE_FACTORS]:
            ts = (amax * factor / 43008.0).float()
            q = lib.empty_quantized(R, C, ts)
            lib.quantize_blockscale(x, ts, rnd, sr_seed(5), 0, row=q)
            lib.dequantize(q, out)
            sc = q.scales
            err = torch.linalg.vector_norm(out - xf) / torch.linalg.vector_norm(xf)
            blk_err = torch.linalg.vector_norm((out - xf).view(R, C // 16, 16), dim=2)
            blk_rel = (blk_err / torch.linalg.vector_norm(xf.view(R, C // 16, 16), dim=2))[blk_nonzero]
            entry[label] = {
                "flushed_frac": round(float(((sc == 0) & blk_nonzero).float().mean()), 5),
                "subnormal_scale_frac": round(float(((sc > 0) & (sc < 8)).float().mean()), 5),
                "saturated_frac": round(float((sc == 0xFE).float().mean()), 6),
                "rel_l2_error": round(float(err), 5),
                "block_rel_error_mean": round(float(blk_rel.mean()), 5),
                "block_rel_error_median": round(float(blk_rel.median()), 5),
            }
        res[name] = entry
    return res


def _event_ms(torch, fn, reps, warm=2):
    """Mean ms per call of fn() over `reps` back-to-back calls (HIP events on
    the current stream, after `warm` untimed calls)."""
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _graph_us(torch, fn, reps):
    """Mean us per replay of fn(0) captured once as a HIP graph
    (torch.cuda.graph), or a string when capture is unavailable."""
    try:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn(0)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    except Exception as ex:  # capture unsupported by this runtime: report, do not fail the run
        return f"unavailable: {type(ex).__name__}: {ex}"[:200]


def config1_latency(lib, torch):
    """The tiny linear (X and W 256 x 256 ~N(0,1) from seed 0, tensor scales
    refreshed from their own amax, round to nearest): one pass of the path --
    amax pass and refresh per tensor, row-wise quantization of X and W,
    fprop (7 launches) -- timed on the GPU with HIP events (latency-bound,
    no roofline claim), eagerly and as replays of the pass captured once as
    a HIP graph (whose output must equal the eager pass's), and the oracle's
    seconds for the same pass on the host."""
    import numpy as np

    from oracle import gemm, quantize, tensor_scale
    from workloads import config

    d = config(1)
    xs = {k: torch.from_numpy(v.view("int16")).cuda() for k, v in d.items()}
    ts = {k: torch.ones(1, dtype=torch.float32, device="cuda") for k in d}
    am = {k: torch.zeros(1, dtype=torch.float32, device="cuda") for k in d}
    q = {k: lib.empty_quantized(256, 256, ts[k]) for k in d}
    y = torch.empty((256, 256), dtype=torch.float32, device="cuda")

    def one_pass(_):
        for k in ("X", "W"):
            lib.quantize_blockscale(xs[k], None, amax=am[k])
            lib.update_tensor_scale(am[k], ts[k], 0, 1)
            lib.quantize_blockscale(xs[k], ts[k], lib.RNE, row=q[k])
        lib.gemm_fprop(q["X"], q["W"], y)

    ms = _event_ms(torch, one_pass, 50, warm=5)
    y_eager = y.clone()
    graph = _graph_us(torch, one_pass, 50)
    if isinstance(graph, float):
        graph = {"gpu_us_per_pass": round(graph, 2), "output_equals_eager": bool(torch.equal(y, y_eager))}
    t0 = time.perf_counter()
    ops = {}
    for k in ("X", "W"):
        _, tsk = tensor_scale.update_tensor_scale(quantize.tensor_amax(d[k]), np.float32(1.0), 0, 1)
        ops[k] = quantize.quantize_blockscale(d[k], tsk, quantize.RNE) + (tsk,)
    gemm.gemm_nt(*ops["X"], *ops["W"])
    oracle_s = time.perf_counter() - t0
    return {"workload": "X, W 256x256 ~N(0,1) seed 0: amax + refresh + RNE row-wise quantize of X and W, "
                        "fprop 256x256x256",
            "gpu_us_per_pass": round(ms * 1e3, 2), "launches_per_pass": 7, "graph_replay": graph,
            "oracle_s_per_pass": round(oracle_s, 4), "bound": "latency"}


def linear_layer_timing(lib, torch, n, stale=None, reps=10, sets=4):
    """One linear layer's hot path on config n's tensors (X, W, dY), call by
    call: the quantization of each tensor (both orientations, amax on; RNE
    for X and W, stochastic rounding for dY) in algorithmic GB/s, and fprop /
    dgrad / wgrad in TFLOP/s.  Tensor scales come from a step-0 refresh of
    each tensor's own amax, multiplied by `stale` when given (a scale from a
    prior step's amax that is off by that factor).  Quantizer inputs and
    outputs rotate over `sets` HBM-resident copies, so each call reads and
    writes HBM rather than the 256 MB cache."""
    from workloads import config, sr_seed

    d = config(n)
    T = {}
    for tid, (name, rnd) in enumerate((("X", lib.RNE), ("W", lib.RNE), ("dY", lib.SR))):
        t = Tensor(lib, torch, d[name], rnd, tid)
        lib.quantize_blockscale(t.x, None, amax=t.amax)
        if stale:
            t.amax.mul_(stale)
        lib.update_tensor_scale(t.amax, t.ts, 0, 1)
        T[name] = t
    del d
    X, W, D = T["X"], T["W"], T["dY"]
    tokens, in_f = X.row.rows, X.row.cols
    out_f = W.row.rows
    res = {"workload": f"config {n}: tokens {tokens}, in {in_f}, out {out_f}"
                       + (f", tensor scales from an amax off by x{stale:g}" if stale else ""),
           "quantize_peak_GBps": HBM_PEAK_GBS, "gemm_peak_TFLOPs": FP16_MFMA_PEAK_TFLOPS}
    for name, t in T.items():
        copies = [(t.x.clone(), lib.empty_quantized(t.row.rows, t.row.cols, t.ts),
                   lib.empty_quantized(t.col.rows, t.col.cols, t.ts)) for _ in range(sets)]

        def quant(i, t=t, copies=copies):
            x, qr, qc = copies[i % len(copies)]
            lib.quantize_blockscale(x, t.ts, t.rounding, sr_seed(n), i, row=qr, col=qc, amax=t.amax)

        ms = _event_ms(torch, quant, reps * sets)
        gbs = t.elems * QUANT_BYTES_PER_ELEM / (ms * 1e-3) / 1e9
        res[f"quantize_{name}"] = {"rounding": "sr" if t.rounding == lib.SR else "rne",
                                   "us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
                                   "frac": round(gbs / HBM_PEAK_GBS, 4)}
        del copies
    Y = torch.empty((tokens, out_f), dtype=torch.float32, device="cuda")
    dX = torch.empty((tokens, in_f), dtype=torch.float32, device="cuda")
    dW = torch.empty((out_f, in_f), dtype=torch.float32, device="cuda")
    for name, fn, a, b, c in (("fprop", lib.gemm_fprop, X.row, W.row, Y),
                              ("dgrad", lib.gemm_dgrad, D.row, W.col, dX),
                              ("wgrad", lib.gemm_wgrad, D.col, X.col, dW)):
        flop = 2.0 * c.shape[0] * c.shape[1] * a.cols
        ms = _event_ms(torch, lambda i, fn=fn, a=a, b=b, c=c: fn(a, b, c), reps)
        tf = flop / (ms * 1e-3) / 1e12
        res[name] = {"shape_MxNxK": f"{c.shape[0]}x{c.shape[1]}x{a.cols}", "us": round(ms * 1e3, 1),
                     "TFLOPs": round(tf, 1), "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}
    del T, Y, dX, dW
    torch.cuda.empty_cache()
    return res


def quantize_only(lib, torch):
    """The quantizer alone on the 8192 x 4096 heavy-tailed activation workload
    (Student-t x normal body, 16 outlier columns x100): row-wise only and
    row-wise + transposed, round-to-nearest and stochastic, tensor amax on;
    the current-tensor-scaling variant (amax pass + scale + quantize); and
    the 2-D (16 x 16 tile) variant, both outputs from one rounding.
    8 device copies of the input and 8 output sets rotate (about 840 MB) so
    every launch reads and writes HBM, not the 256 MB cache.  GB/s counts the
    algorithmic bytes: 2 per element read, 0.5625 per element per output.
    The streaming reference (a kernel that moves the same bytes as contiguous
    streams, no quantization) is timed on the same buffers: each variant's
    frac_of_stream_reference is its time against that, the share of the HBM
    rate its read/write mix can reach that it reaches."""
    from workloads import config, sr_seed

    bits = config(2)["X"]
    rows, cols = bits.shape
    sets = 8
    x0 = torch.from_numpy(bits.view("int16")).cuda()
    xs = [x0.clone() for _ in range(sets)]
    del x0
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    lib.quantize_blockscale(xs[0], None, amax=amax)
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    lib.update_tensor_scale(amax, ts, 0, 1)
    outs = [(lib.empty_quantized(rows, cols, ts), lib.empty_quantized(cols, rows, ts)) for _ in range(sets)]
    iters = 40
    res = {"workload": f"activations {rows}x{cols} bf16 (heavy-tailed, outlier columns)",
           "peak": HBM_PEAK_GBS, "unit": "GB/s", "buffer_sets": sets}
    ts_cur = torch.ones(1, dtype=torch.float32, device="cuda")
    for name, rnd, both, current in (("rne_row", lib.RNE, False, False),
                                     ("rne_row_col", lib.RNE, True, False),
                                     ("sr_row", lib.SR, False, False),
                                     ("sr_row_col", lib.SR, True, False),
                                     ("current_scaling_rne_row_col", lib.RNE, True, True),
                                     ("tile2d_rne_row_col", lib.RNE, True, False),
                                     ("tile2d_sr_row_col", lib.SR, True, False),
                                     ("stream_reference_row", None, False, False),
                                     ("stream_reference_row_col", None, True, False)):
        def run(i):
            k = i % sets
            if name.startswith("stream_reference"):
                lib.stream_reference(xs[k], outs[k][0], outs[k][1] if both else None)
            elif name.startswith("tile2d"):
                lib.quantize_blockscale_2d(xs[k], ts, rnd, sr_seed(2), i, row=outs[k][0], col=outs[k][1],
                                           amax=amax)
            elif current:
                lib.quantize_current_scaling(xs[k], ts_cur, amax, rnd, sr_seed(2), i, row=outs[k][0],
                                             col=outs[k][1] if both else None)
            else:
                lib.quantize_blockscale(xs[k], ts, rnd, sr_seed(2), i, row=outs[k][0],
                                        col=outs[k][1] if both else None, amax=amax)
        for i in range(sets):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        nbytes = rows * cols * (2 + 0.5625 * (2 if both else 1))
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes": nbytes}
    # current-tensor scaling reads x twice (amax pass, then quantization):
    # its GB/s above counts the periodic path's algorithmic bytes, so the
    # ratio of times is the cost of the extra pass that periodic scaling saves
    cur = res["current_scaling_rne_row_col"]
    cur["extra_read_bytes"] = rows * cols * 2
    cur["time_vs_periodic"] = round(cur["us"] / res["rne_row_col"]["us"], 3)
    for name, r in res.items():
        if isinstance(r, dict) and not name.startswith("stream_reference"):
            ref = res["stream_reference_row_col" if "row_col" in name else "stream_reference_row"]
            r["frac_of_stream_reference"] = round(ref["us"] / r["us"], 4)
    return res


def cpu_baseline(step_flops, step_elems, sample):
    """The CPU oracle (as it stands) on a bounded sample of one step, about
    10-20 s of host work: the stochastic-rounding quantization of 3072 output
    rows of dY_up in each orientation (numpy, one thread) and the fp64 GEMM
    of 4096 output rows of the up projection's fprop (numpy matmul on the
    BLAS threads, dequantization and the tolerance bound included).  The
    step time is extrapolated per output element and per flop and reported in
    the same TFLOP/s unit as `value`.  `cores` is the largest number of
    threads the sample ran on (the BLAS pool); the host's CPU count and the
    process's affinity mask are recorded beside it."""
    import numpy as np

    from oracle import gemm, quantize
    from workloads import sr_seed

    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    affinity = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    dy = sample["dY_up"]
    t0 = time.perf_counter()
    for o, n_out in ((0, dy.shape[0]), (1, dy.shape[1])):
        rows = np.arange(CPU_QUANT_ROWS) * (n_out // CPU_QUANT_ROWS)
        quantize.quantize_blockscale(dy, np.float32(1e-7), quantize.SR, sr_seed(4), 0, o, rows=rows)
    tq = time.perf_counter() - t0
    q_elems = CPU_QUANT_ROWS * dy.shape[1] + CPU_QUANT_ROWS * dy.shape[0]  # output elements produced
    x, w = sample["X_rows"], sample["W_up"]
    xc, xs = quantize.quantize_blockscale(x, np.float32(1e-4), quantize.RNE)
    wc, ws = quantize.quantize_blockscale(w, np.float32(1e-6), quantize.RNE)
    t1 = time.perf_counter()
    gemm.gemm_nt(xc, xs, 1e-4, wc, ws, 1e-6)
    tg = time.perf_counter() - t1
    g_flops = 2.0 * x.shape[0] * w.shape[0] * w.shape[1]
    # every input element is quantized in two orientations per step
    est_step_s = tq / q_elems * (2 * step_elems) + tg / g_flops * step_flops
    return {"value": round(step_flops / est_step_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(blas), "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "affinity_cpus": len(affinity),
            "affinity_mask": _cpu_ranges(affinity),
            "quantize_threads": 1, "gemm_threads": int(blas),
            "quantize_GBps": round(q_elems * 3.125 / 2 / tq / 1e9, 4),
            "gemm_GFLOPs": round(g_flops / tg / 1e9, 2),
            "sample": f"quantize (SR) of {CPU_QUANT_ROWS} output rows per orientation of dY_up "
                      f"8192x16384 ({tq:.1f} s, 1 thread) + fp64 fprop GEMM of {x.shape[0]} x 16384 x "
                      f"4096 ({tg:.1f} s, {blas} BLAS threads, dequantize and bound included); step "
                      f"time extrapolated per element and per flop: {est_step_s:.0f} s"}


def _cpu_ranges(cpus):
    """[0, 1, 2, 5] -> '0-2,5'."""
    out, start, prev = [], None, None
    for c in cpus:
        if start is None:
            start = prev = c
        elif c == prev + 1:
            prev = c
        else:
            out.append(f"{start}-{prev}" if prev > start else str(start))
            start = prev = c
    if start is not None:
        out.append(f"{start}-{prev}" if prev > start else str(start))
    return ",".join(out)


if __name__ == "__main__":
    main()

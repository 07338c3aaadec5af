#!/usr/bin/env python3
"""Throughput of one MoE layer step (schedule + forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer over one batch of synthetic input:
top-k routing and the schedule, dispatch, the expert-grouped SwiGLU FFN and
the weighted combine, then the backward (reverse-combine, SwiGLU backward with
the router-weight gradient, expert dgrad/wgrad, reverse-dispatch, softmax
backward).  Inputs are resident in HBM before timing starts.

FLOPs per step follow the usual MoE convention: 6*H*I per routed token-slot
forward and 12*H*I backward (routing, softmax and elementwise work excluded).

Prints one JSON line.  It carries the layer throughput (also as a fraction of
the MFMA peak), a roofline entry for the kernel with the largest share of the
step (its algorithmic bytes per launch over its average duration, timed with
HIP events on the launch stream), the whole step against HBM (the algorithmic
bytes of all its launches over 8 TB/s), and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

WORKLOADS = ("e512_t2048", "e512_t65536_zipf", "e8_ep_share")
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}    # MI355X dense matrix peaks
PAGES_CONTEXT = ("MoK 531.1 and HybridEP + Megatron 224.4 TFLOP/s per GPU: MXFP8 forward of the "
                 "512-expert H=4096 I=1024 top-10 layer on 64 GB300 GPUs (expert parallelism 64, "
                 "cross-GPU dispatch/combine included); other hardware and setup, so vs_baseline is null")

# HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE on e512_t2048,
# each scaled by what that counter reads for a copy kernel of known size
# (FETCH_SIZE counts half of a copy's reads: x2; WRITE_SIZE counts them all);
# filled in from profiles/, and dropped whenever the kernel changes.
TRAFFIC = {                      # profiles/kernels_e512_t2048.txt
    "gemm_gate_up": 8888.0e6,
    "gemm_gu_dgrad": 8882.0e6,
    "wgrad_gate_up": 8825.7e6,
    "gemm_down": 4505.6e6,
    "gemm_down_dgrad": 4690.2e6,
    "wgrad_down": 4486.0e6,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="e512_t2048", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=48,
                    help="tokens in the CPU oracle's sample (forward + input gradients)")
    ap.add_argument("--cpu-experts", type=int, default=12,
                    help="experts in the CPU oracle's sample (weight gradients)")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the MXFP8 leg (reported beside the bf16 value)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only time plain HBM copy / fill / read kernels of known size and exit")
    return ap.parse_args()


def calibrate(torch, nbytes=4 << 30, reps=10):
    """Bandwidth of plain torch copy, fill and sum kernels on buffers of known size."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    out = {}
    for name, fn, moved in (("copy", lambda: b.copy_(a), 2 * nbytes),
                            ("fill", lambda: b.fill_(1.0), nbytes),
                            ("sum", lambda: a.sum(dtype=torch.float32), nbytes)):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        out[name] = {"bytes": moved, "avg_ms": round(ms, 4), "GB/s": round(moved / ms / 1e6, 1)}
    return out


def kernel_bytes(shape, counts: np.ndarray) -> dict:
    """Algorithmic HBM bytes per launch of each kernel (the unique data it must
    move) for a workload that fits one macrobatch.  With several macrobatches
    the per-launch figures differ per launch, and none are given."""
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    if shape.macrobatch and shape.macrobatch < T:
        return {}
    S = T * k
    used = int(np.count_nonzero(counts))
    P = I // 128
    w_gu = used * 2 * I * H * 2
    w_d = used * H * I * 2
    q = 1 + 1 / 32                      # an MXFP8 code and its share of a scale byte
    return {
        "topk_route": T * E * 4 + S * 8,
        "dispatch": T * H * 2 + S * H * 2,
        "gemm_gate_up": w_gu + S * H * 2 + 3 * S * I * 2,
        "gemm_down": w_d + S * I * 2 + S * H * 2,
        "combine": S * H * 2 + T * H * 2 + S * 8,
        "gemm_down_dgrad": w_d + T * H * 2 + 2 * S * I * 2 + 3 * S * I * 2 + S * P * 4,
        "gemm_gu_dgrad": w_gu + S * 2 * I * 2 + S * H * 2,
        "wgrad_down": E * H * I * 2 + T * H * 2 + S * I * 2,
        "wgrad_gate_up": E * 2 * I * H * 2 + T * H * 2 + S * 2 * I * 2,
        "rd_reduce": S * H * 2 + T * H * 2,
        "softmax_bwd": S * P * 4 + T * E * 4 + S * 12,
        # MXFP8 leg
        "dispatch_mx": T * H * 2 + S * H * q,
        "gemm_gate_up_mx": int(w_gu / 2 * q + S * H * q + 2 * S * I * 4 + S * I * q),
        "gemm_down_mx": int(w_d / 2 * q + S * I * q + S * H * 2),
        "gemm_down_dgrad_mx": int(w_d / 2 * q + T * H * q + 4 * S * I * 4 + S * I * 4
                                  + 2 * S * I * q + S * P * 4),
        "gemm_gu_dgrad_mx": int(w_gu / 2 * q + 2 * S * I * q + S * H * 2),
        "wgrad_down_mx": int(E * H * I * 2 + (H + I) * S * q),
        "wgrad_gate_up_mx": int(E * 2 * I * H * 2 + (2 * I + H) * S * q),
        "mx_quant_rows": int(T * H * 2 + T * H * q),
        "mx_qt_wdy": int(T * H * 2 + S * H * q),
        "mx_qt_x": int(T * H * 2 + S * H * q),
        "mx_qt_f32": int((3 * S * I * 4 + 3 * S * I * q) / 2),   # mean of its two launches
    }


def kernel_flops(shape) -> dict:
    """Matrix flops per step of each GEMM launcher (all its launches), by the
    6 H I per row forward / 12 H I backward convention split over the GEMMs."""
    rows = shape.T * shape.k + (shape.T if shape.n_shared else 0)
    f = 2.0 * shape.H * shape.I * rows
    out = {"gemm_gate_up": 2 * f, "gemm_down": f, "gemm_down_dgrad": f, "gemm_gu_dgrad": 2 * f,
           "wgrad_down": f, "wgrad_gate_up": 2 * f}
    out.update({k + "_mx": v for k, v in list(out.items())})
    return out


def cpu_baseline(case, idx, w, n_tokens: int, n_experts: int):
    """Time the oracle on a bounded sample of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info

    shape = case.shape
    H, I, k = shape.H, shape.I, shape.k
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(shape.T, size=n_tokens, replace=False))
    counts = np.bincount(idx.reshape(-1), minlength=shape.E)
    experts = [int(e) for e in rng.choice(np.nonzero(counts)[0], size=n_experts, replace=False)]
    need = sorted(set(idx[tokens].reshape(-1).tolist()) | set(experts))
    # host copies of the weights the sample touches (fetched before timing)
    wg = {e: case.wg[e].float().cpu().numpy() for e in need}
    wu = {e: case.wu[e].float().cpu().numpy() for e in need}
    wd = {e: case.wd[e].float().cpu().numpy() for e in need}
    x = case.x.float().cpu().numpy()
    dy = case.dy.float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.forward(x, wg, wu, wd, idx, w, tokens=tokens)
    oracle.backward(x, wg, wu, wd, idx, w, dy, tokens=tokens, experts=experts)
    dt = time.perf_counter() - t0
    rows = int(sum(counts[e] for e in experts))
    flops = 12.0 * H * I * k * n_tokens + 6.0 * H * I * rows
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle: forward + input-gradient backward of {n_tokens} tokens "
                   f"({n_tokens * k} slots) and the weight gradients of {n_experts} experts "
                   f"({rows} rows) of the {shape.name} workload; {dt:.1f} s"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer is "
              "built for a single MI355X and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth_inputs as si
    from mixture_experts_layer_dispatch_amd import binding as B

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if not B.device_supported():
        print("the library requires gfx950 (MI355X)", file=sys.stderr)
        sys.exit(1)
    if args.calibrate:
        print(json.dumps({"hbm_calibration": calibrate(torch)}), flush=True)
        return

    shape = si.SHAPES[args.workload]
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    cfg = B.Config(T=T, H=H, I=I, E=E, k=k, n_shared=shape.n_shared,
                   macrobatch=shape.macrobatch, minibatch=shape.minibatch)

    class Case:
        pass

    case = Case()
    case.shape = shape
    case.logits = si.logits(shape, "cuda")
    case.x = si.tokens(shape, "cuda")
    case.dy = si.grad_out(shape, "cuda")
    case.wg, case.wu, case.wd = si.all_expert_weights(shape, "cuda")
    weights = {"w_gate": case.wg, "w_up": case.wu, "w_down": case.wd}
    shared = si.shared_weights(shape, "cuda")
    if shared is not None:
        weights.update({"s_gate": shared[0], "s_up": shared[1], "s_down": shared[2]})
    sched = B.alloc_schedule(cfg)
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    dw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    dlog = torch.empty(T, E, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    S = T * k
    flops = 18.0 * H * I * S + (18.0 * H * I * T if shape.n_shared else 0.0)
    flops_fwd = flops / 3.0

    def run(precision):
        """Time K steps of schedule + forward + backward, then a second pass with
        per-kernel HIP events; returns (ms/step, kernel stats)."""
        c = B.Config(T=T, H=H, I=I, E=E, k=k, n_shared=shape.n_shared,
                     macrobatch=shape.macrobatch, minibatch=shape.minibatch, precision=precision)
        ws = B.alloc_workspace(c)
        saved = B.alloc_saved(c)
        grads = B.alloc_grads(c)
        wts = dict(weights)
        if precision == B.PREC_MXFP8:
            q = B.alloc_weights_mx(c)
            B.moe_quantize_weights_mxfp8(c, weights, q, stream)   # outside timing
            wts["mx"] = q

        def step():
            B.moe_schedule(c, case.logits, sched, ws, stream)
            B.moe_forward(c, sched, case.x, wts, y, saved, ws, stream)
            B.moe_backward(c, sched, saved, case.x, wts, case.dy, dx, grads, dw, dlog, ws, stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
        # forward alone (the schedule of the last step stays in place), the
        # form in which the pages quote their MXFP8 numbers
        start.record(stream)
        for _ in range(args.steps):
            B.moe_forward(c, sched, case.x, wts, y, saved, ws, stream)
        stop.record(stream)
        torch.cuda.synchronize()
        ms_fwd = start.elapsed_time(stop) / args.steps
        assert B.moe_check_device_error(ws, stream) == 0
        B.profile_reset()
        B.profile_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        B.profile_collect()
        B.profile_enable(False)
        stats = B.profile_stats()
        del ws, saved, grads, wts
        return ms, ms_fwd, stats

    ms, ms_fwd, stats = run(B.PREC_BF16)
    print(f"[bench] bf16: {args.steps} steps, {ms:.3f} ms/step", file=sys.stderr, flush=True)
    value = flops / (ms * 1e-3) / 1e12
    counts = sched["counts"].cpu().numpy().sum(0)
    kb = kernel_bytes(shape, counts)

    def kernel_table(st):
        out = {}
        for name, (n, tot) in st.items():
            avg = tot / max(n, 1)
            entry = {"launches_per_step": n / args.steps, "avg_ms": round(avg, 4)}
            if name in kb:
                entry["GB/s"] = round(kb[name] / (avg * 1e-3) / 1e9, 1)
            out[name] = entry
        return out

    def step_roofline(st, ms_step):
        """The whole step against HBM: the algorithmic bytes of every launch
        over 8 TB/s is the step's floor; frac = floor / measured."""
        if not kb:
            return None
        tot = sum(kb[n] * cnt / args.steps for n, (cnt, _) in st.items() if n in kb)
        floor = tot / (HBM_PEAK_GBS * 1e9) * 1e3
        return {"bound": "hbm", "algorithmic_bytes": int(tot), "floor_ms": round(floor, 4),
                "frac": round(floor / ms_step, 4),
                "TFLOP/s_ceiling": round(flops / (floor * 1e-3) / 1e12, 1)}

    kernels = kernel_table(stats)
    dom = max(stats, key=lambda n: stats[n][1])
    dom_avg = stats[dom][1] / stats[dom][0]
    kf = kernel_flops(shape)
    ridge = MFMA_PEAK_TFLOPS["bf16"] * 1e12 / (HBM_PEAK_GBS * 1e9)     # flop per byte
    roofline = None
    per_step = stats[dom][0] / args.steps                  # launches of the kernel per step
    if dom in kb and (dom not in kf or kf[dom] / (kb[dom] * per_step) < ridge):
        achieved = kb[dom] / (dom_avg * 1e-3) / 1e9
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": TRAFFIC.get(dom) if args.workload == "e512_t2048" else None,
                    "avg_ms": round(dom_avg, 4), "bytes_per_launch": kb[dom]}
    elif dom in kf:
        # a GEMM whose groups are large (or a stream of macrobatches, where
        # per-launch bytes are not given): against the matrix peak, over all
        # of its launches in a step
        achieved = kf[dom] / (stats[dom][1] / args.steps * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_PEAK_TFLOPS["bf16"], 4), "traffic": None,
                    "avg_ms": round(dom_avg, 4), "launches_per_step": per_step,
                    "flops_per_step": kf[dom]}

    mx = None
    if not args.no_mxfp8:
        ms_mx, ms_fwd_mx, stats_mx = run(B.PREC_MXFP8)
        print(f"[bench] mxfp8: {args.steps} steps, {ms_mx:.3f} ms/step", file=sys.stderr, flush=True)
        v_mx = flops / (ms_mx * 1e-3) / 1e12
        mx = {"value": round(v_mx, 2), "unit": "TFLOP/s",
              "mfma_peak_frac": round(v_mx / MFMA_PEAK_TFLOPS["mxfp8"], 4),
              "ms_per_step": round(ms_mx, 4), "dtype": "mxfp8 (e4m3 + e8m0 per 32)",
              "step_roofline": step_roofline(stats_mx, ms_mx),
              "forward": {"ms": round(ms_fwd_mx, 4),
                          "TFLOP/s": round(flops_fwd / (ms_fwd_mx * 1e-3) / 1e12, 2)},
              "kernels": kernel_table(stats_mx)}

    cpu = None
    if not args.no_cpu_baseline:
        idx = sched["topk_idx"].cpu().numpy()
        wts = sched["topk_w"].cpu().numpy().astype(np.float64)
        import oracle  # noqa: F401  (test infrastructure: the CPU baseline only)
        cpu = cpu_baseline(case, idx, wts, args.cpu_tokens, args.cpu_experts)

    out = {
        "metric": "MoE layer TFLOP/s fwd+bwd (bf16, MXFP8) at 512E H4096 I1024 top-10",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: T={T} H={H} I={I} E={E} top-{k}, bf16, "
                               "schedule+forward+backward",
                   "T": T, "H": H, "I": I, "E": E, "k": k, "parallelism": "none (1 GPU)"},
        "mfma_peak_frac": round(value / MFMA_PEAK_TFLOPS["bf16"], 4),
        "forward": {"ms": round(ms_fwd, 4), "TFLOP/s": round(flops_fwd / (ms_fwd * 1e-3) / 1e12, 2)},
        "roofline": roofline,
        "step_roofline": step_roofline(stats, ms),
        "pages_context": PAGES_CONTEXT,
        "cpu_baseline": cpu,
        "mxfp8": mx,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

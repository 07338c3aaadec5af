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

ROOT = os.path.dirname(os.path.abspath(__file__))


def counter_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from rocprofv3 FETCH_SIZE + WRITE_SIZE
    runs (each scaled by what that counter reads for a copy kernel of known
    size), as recorded in profiles/traffic_<workload>.json, with the state of
    the record: "measured" when the file's source hash matches the HIP sources
    of this build, else "stale" (the kernels changed since: bytes None) or
    "absent"."""
    from mixture_experts_layer_dispatch_amd.prof_summary import sources_sha256

    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, "absent"
    rec = json.load(open(path))
    if rec.get("sources_sha256") != sources_sha256():
        return None, "stale"
    k = rec.get("kernels", {}).get("k_" + kernel)
    if k is None:
        return None, "absent"
    return k["read_bytes"] + k["write_bytes"], "measured"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="e512_t2048", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=24,
                    help="tokens in the CPU oracle's sample (forward + input gradients)")
    ap.add_argument("--cpu-experts", type=int, default=6,
                    help="experts in the CPU oracle's sample (weight gradients)")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the MXFP8 leg (reported beside the bf16 value)")
    ap.add_argument("--no-ep-share", action="store_true",
                    help="skip the expert-parallel-share leg (reported beside the headline)")
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
        # the dispatch is fused into the gate/up GEMM's loads: x is read once
        # (a token's k rows are re-read from cache), g, u, h written
        "gemm_gate_up": w_gu + T * H * 2 + 3 * S * I * 2,
        "gemm_down": w_d + S * I * 2 + S * H * 2 + S * 8,
        "combine": S * H * 2 + T * H * 2 + S * 4,
        "gemm_down_dgrad": w_d + T * H * 2 + 2 * S * I * 2 + 3 * S * I * 2 + S * P * 4,
        "gemm_gu_dgrad": w_gu + S * 2 * I * 2 + S * H * 2,
        "wgrad_down": E * H * I * 2 + T * H * 2 + S * I * 2,
        "wgrad_gate_up": E * 2 * I * H * 2 + T * H * 2 + S * 2 * I * 2,
        "rd_reduce": S * H * 2 + T * H * 2,
        "softmax_bwd": S * P * 4 + T * E * 4 + S * 12,
        # MXFP8 leg (x quantised once per token by mx_quant_rows, gathered on load)
        "gemm_gate_up_mx": int(w_gu / 2 * q + T * H * q + 2 * S * I * 4 + S * I * q),
        "gemm_down_mx": int(w_d / 2 * q + S * I * q + S * H * 2 + S * 8),
        # g, u read; dg | du quantised along I; h, dg, du quantised along the
        # group's rows and written transposed (the weight gradients' operands)
        "gemm_down_dgrad_mx": int(w_d / 2 * q + T * H * q + 2 * S * I * 4 + 2 * S * I * q
                                  + 3 * S * I * q + S * P * 4),
        "gemm_gu_dgrad_mx": int(w_gu / 2 * q + 2 * S * I * q + S * H * 2),
        "wgrad_down_mx": int(E * H * I * 2 + (H + I) * S * q),
        "wgrad_gate_up_mx": int(E * 2 * I * H * 2 + (2 * I + H) * S * q),
        "mx_quant_rows": int(T * H * 2 + T * H * q),       # x (forward) and dy (backward)
        "mx_qt_wdy": int(T * H * 2 + S * H * q),
        "mx_qt_x": int(T * H * 2 + S * H * q),
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


def cpu_baseline(case, n_tokens: int, n_experts: int):
    """Time the oracle on a bounded sample of the same workload: routing and the
    schedule of the whole batch (its own, from the logits on the host), then the
    forward and input-gradient backward of n_tokens tokens and the weight
    gradients of n_experts experts.  One untimed warm-up run, then the median
    of three timed runs."""
    import oracle
    from threadpoolctl import threadpool_info

    shape = case.shape
    H, I, k = shape.H, shape.I, shape.k
    logits = case.logits.cpu().numpy()
    idx, w = oracle.route(logits, k)
    counts = np.bincount(idx.reshape(-1), minlength=shape.E)
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(shape.T, size=n_tokens, replace=False))
    experts = [int(e) for e in rng.choice(np.nonzero(counts)[0], size=n_experts, replace=False)]
    need = sorted(set(idx[tokens].reshape(-1).tolist()) | set(experts))
    # host copies of the weights the sample touches (fetched before timing)
    wg = {e: case.wg[e].float().cpu().numpy() for e in need}
    wu = {e: case.wu[e].float().cpu().numpy() for e in need}
    wd = {e: case.wd[e].float().cpu().numpy() for e in need}
    x = case.x.float().cpu().numpy()
    dy = case.dy.float().cpu().numpy()

    def once():
        t0 = time.perf_counter()
        idx_, w_ = oracle.route(logits, k)
        oracle.schedule(idx_, shape.E)
        oracle.forward(x, wg, wu, wd, idx_, w_, tokens=tokens)
        oracle.backward(x, wg, wu, wd, idx_, w_, dy, tokens=tokens, experts=experts)
        return time.perf_counter() - t0

    once()
    runs = sorted(once() for _ in range(3))
    dt = runs[1]
    rows = int(sum(counts[e] for e in experts))
    flops = 12.0 * H * I * k * n_tokens + 6.0 * H * I * rows
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle: routing + schedule of all {shape.T} tokens, forward + "
                   f"input-gradient backward of {n_tokens} tokens ({n_tokens * k} slots) and the "
                   f"weight gradients of {n_experts} experts ({rows} rows) of the {shape.name} "
                   f"workload; median of 3 timed runs after 1 warm-up: {dt:.2f} s "
                   f"(runs {', '.join(f'{r:.2f}' for r in runs)} s); flops counted on the sample only"),
    }


class Inputs:
    """Seeded inputs of one workload, resident on the GPU."""

    def __init__(self, si, shape):
        self.shape = shape
        self.logits = si.logits(shape, "cuda")
        self.x = si.tokens(shape, "cuda")
        self.dy = si.grad_out(shape, "cuda")
        self.wg, self.wu, self.wd = si.all_expert_weights(shape, "cuda")
        self.weights = {"w_gate": self.wg, "w_up": self.wu, "w_down": self.wd}
        shared = si.shared_weights(shape, "cuda")
        if shared is not None:
            self.weights.update({"s_gate": shared[0], "s_up": shared[1], "s_down": shared[2]})


def step_flops(shape) -> float:
    """Convention flops of one step: 18 H I per routed slot (+ per token for a
    shared expert); the forward is a third of it."""
    f = 18.0 * shape.H * shape.I * shape.T * shape.k
    return f + (18.0 * shape.H * shape.I * shape.T if shape.n_shared else 0.0)


def measure(torch, B, inp, precision, steps, warmup, stream):
    """Time `steps` steps of schedule + forward + backward (after `warmup`),
    then `steps` forward-only passes, then a pass with per-kernel HIP events.
    Returns (ms per step, ms per forward, kernel stats, per-expert counts)."""
    shape = inp.shape
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    c = B.Config(T=T, H=H, I=I, E=E, k=k, n_shared=shape.n_shared,
                 macrobatch=shape.macrobatch, minibatch=shape.minibatch, precision=precision)
    ws = B.alloc_workspace(c)
    sched = B.alloc_schedule(c)
    saved = B.alloc_saved(c)
    grads = B.alloc_grads(c)
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    dw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    dlog = torch.empty(T, E, dtype=torch.float32, device="cuda")
    wts = dict(inp.weights)
    if precision == B.PREC_MXFP8:
        q = B.alloc_weights_mx(c)
        B.moe_quantize_weights_mxfp8(c, inp.weights, q, stream)   # outside timing
        wts["mx"] = q

    def step():
        B.moe_schedule(c, inp.logits, sched, ws, stream)
        B.moe_forward(c, sched, inp.x, wts, y, saved, ws, stream)
        B.moe_backward(c, sched, saved, inp.x, wts, inp.dy, dx, grads, dw, dlog, ws, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    # forward alone (the schedule of the last step stays in place), the form in
    # which the pages quote their MXFP8 numbers
    start.record(stream)
    for _ in range(steps):
        B.moe_forward(c, sched, inp.x, wts, y, saved, ws, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_fwd = start.elapsed_time(stop) / steps
    assert B.moe_check_device_error(ws, stream) == 0
    B.profile_reset()
    B.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    B.profile_collect()
    B.profile_enable(False)
    stats = B.profile_stats()
    counts = sched["counts"].cpu().numpy().sum(0)
    del ws, saved, grads, wts
    return ms, ms_fwd, stats, counts


def kernel_table(stats, steps, kb):
    out = {}
    for name, (n, tot) in stats.items():
        avg = tot / max(n, 1)
        entry = {"launches_per_step": n / steps, "avg_ms": round(avg, 4)}
        if name in kb:
            entry["GB/s"] = round(kb[name] / (avg * 1e-3) / 1e9, 1)
        out[name] = entry
    return out


def mfma_dominant(stats, steps, shape, prec):
    """The GEMM with the largest time per step, as a fraction of the dense
    matrix peak of its precision: its convention flops per step (its share of
    the step's flops) over its measured time per step."""
    kf = kernel_flops(shape)
    gem = {n: v for n, v in stats.items() if n in kf}
    if not gem:
        return None
    dom = max(gem, key=lambda n: gem[n][1])
    t = gem[dom][1] / steps
    tf = kf[dom] / (t * 1e-3) / 1e12
    return {"kernel": dom, "ms_per_step": round(t, 4), "TFLOP/s": round(tf, 1),
            "mfma_frac": round(tf / MFMA_PEAK_TFLOPS[prec], 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer is "
              "built for a single MI355X and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, ROOT)
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
    inp = Inputs(si, shape)
    stream = torch.cuda.current_stream()
    flops = step_flops(shape)
    flops_fwd = flops / 3.0

    ms, ms_fwd, stats, counts = measure(torch, B, inp, B.PREC_BF16, args.steps, args.warmup, stream)
    print(f"[bench] bf16: {args.steps} steps, {ms:.3f} ms/step", file=sys.stderr, flush=True)
    value = flops / (ms * 1e-3) / 1e12
    kb = kernel_bytes(shape, counts)

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

    kernels = kernel_table(stats, args.steps, kb)
    dom = max(stats, key=lambda n: stats[n][1])
    dom_avg = stats[dom][1] / stats[dom][0]
    kf = kernel_flops(shape)
    ridge = MFMA_PEAK_TFLOPS["bf16"] * 1e12 / (HBM_PEAK_GBS * 1e9)     # flop per byte
    roofline = None
    per_step = stats[dom][0] / args.steps                  # launches of the kernel per step
    if dom in kb and (dom not in kf or kf[dom] / (kb[dom] * per_step) < ridge):
        achieved = kb[dom] / (dom_avg * 1e-3) / 1e9
        traffic, tstate = counter_traffic(args.workload, dom)
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "traffic_source": tstate,
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
        ms_mx, ms_fwd_mx, stats_mx, _ = measure(torch, B, inp, B.PREC_MXFP8, args.steps,
                                                args.warmup, stream)
        print(f"[bench] mxfp8: {args.steps} steps, {ms_mx:.3f} ms/step", file=sys.stderr, flush=True)
        v_mx = flops / (ms_mx * 1e-3) / 1e12
        mx = {"value": round(v_mx, 2), "unit": "TFLOP/s",
              "mfma_peak_frac": round(v_mx / MFMA_PEAK_TFLOPS["mxfp8"], 4),
              "ms_per_step": round(ms_mx, 4), "dtype": "mxfp8 (e4m3 + e8m0 per 32)",
              "step_roofline": step_roofline(stats_mx, ms_mx),
              "forward": {"ms": round(ms_fwd_mx, 4),
                          "TFLOP/s": round(flops_fwd / (ms_fwd_mx * 1e-3) / 1e12, 2)},
              "kernels": kernel_table(stats_mx, args.steps, kb)}

    w4 = None
    if not args.no_mxfp8:
        # the MXFP4-weight forward (E2M1 weights, MXFP8 activations; forward
        # only): the weight stream of the forward halves against MXFP8
        c4 = B.Config(T=T, H=H, I=I, E=E, k=k, n_shared=shape.n_shared, macrobatch=shape.macrobatch,
                      minibatch=shape.minibatch, precision=B.PREC_MXFP4)
        ws4 = B.alloc_workspace(c4)
        sch4 = B.alloc_schedule(c4)
        sv4 = B.alloc_saved(c4)
        q4 = B.alloc_weights_mx4(c4)
        B.moe_quantize_weights_mxfp4(c4, inp.weights, q4, stream)      # outside timing
        wts4 = dict(inp.weights, mx4=q4)
        y4 = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        B.moe_schedule(c4, inp.logits, sch4, ws4, stream)
        for _ in range(args.warmup):
            B.moe_forward(c4, sch4, inp.x, wts4, y4, sv4, ws4, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            B.moe_forward(c4, sch4, inp.x, wts4, y4, sv4, ws4, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms4 = e0.elapsed_time(e1) / args.steps
        w4 = {"ms": round(ms4, 4), "TFLOP/s": round(flops_fwd / (ms4 * 1e-3) / 1e12, 2),
              "dtype": "weights mxfp4 (e2m1 + e8m0 per 32), activations mxfp8; forward only"}
        print(f"[bench] mxfp4-weight forward: {ms4:.3f} ms", file=sys.stderr, flush=True)
        del ws4, sv4, q4, wts4, y4

    router = None
    if shape.E <= 1024:
        # the router projection upstream of the layer (outside the metric, as on
        # the pages): logits = x W_r^T, and its backward
        wr = si.router_weights(shape, "cuda")
        lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
        dxr = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
        dwr = torch.empty(E, H, dtype=torch.bfloat16, device="cuda")
        cr = B.Config(T=T, H=H, I=I, E=E, k=k, n_shared=shape.n_shared, macrobatch=shape.macrobatch,
                      minibatch=shape.minibatch)
        wsr = B.alloc_workspace(cr)

        def rstep():
            B.moe_router_forward(cr, inp.x, wr, lg, stream)
            B.moe_router_backward(cr, inp.x, wr, lg, dxr, dwr, wsr, stream)

        for _ in range(args.warmup):
            rstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            rstep()
        e1.record(stream)
        torch.cuda.synchronize()
        msr = e0.elapsed_time(e1) / args.steps
        rfl = 3 * 2.0 * T * H * E
        router = {"ms_fwd_bwd": round(msr, 4), "TFLOP/s": round(rfl / (msr * 1e-3) / 1e12, 1),
                  "note": "router projection x W_r^T and its backward (d_logits W_r into dx, dW_r); "
                          "outside the layer metric"}
        del wr, lg, dxr, dwr, wsr

    ep = None
    if not args.no_ep_share and args.workload != "e8_ep_share":
        # one GPU's expert-parallel share (8 experts x 2560 rows): the MFMA-bound
        # shape of the same layer, measured beside the headline
        es = si.SHAPES["e8_ep_share"]
        einp = Inputs(si, es)
        ef = step_flops(es)
        ep = {"workload": f"{es.name}: T={es.T} rows H={es.H} I={es.I} E={es.E} top-{es.k}, "
                          "schedule+forward+backward", "steps": 10, "warmup": 3}
        for prec, pname in ((B.PREC_BF16, "bf16"), (B.PREC_MXFP8, "mxfp8")):
            if prec == B.PREC_MXFP8 and args.no_mxfp8:
                continue
            e_ms, e_fwd, e_st, _ = measure(torch, B, einp, prec, 10, 3, stream)
            tf = ef / (e_ms * 1e-3) / 1e12
            ep[pname] = {"TFLOP/s": round(tf, 1), "ms_per_step": round(e_ms, 4),
                         "mfma_peak_frac": round(tf / MFMA_PEAK_TFLOPS[pname], 4),
                         "forward": {"ms": round(e_fwd, 4),
                                     "TFLOP/s": round(ef / 3 / (e_fwd * 1e-3) / 1e12, 1)},
                         "dominant": mfma_dominant(e_st, 10, es, pname),
                         "kernels": kernel_table(e_st, 10, {})}
            print(f"[bench] ep_share {pname}: {e_ms:.3f} ms/step", file=sys.stderr, flush=True)
        del einp

    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # noqa: F401  (test infrastructure: the CPU baseline only)
        cpu = cpu_baseline(inp, args.cpu_tokens, args.cpu_experts)

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
        "mxfp4_weight_forward": w4,
        "router": router,
        "ep_share": ep,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

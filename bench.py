#!/usr/bin/env python3
"""Throughput of the attention backward on one MI355X.

Workload: causal, bf16, B=2, H=32, n=m=4096, d=dv=128, seed 2, scale
1/sqrt(128).  A step is one backward pass (D preprocess, dK/dV kernel, dQ
kernel) over inputs already resident in HBM; O and LSE come from the
forward kernel, which runs before the timed region and is timed on its own
as context.  FLOPs follow the convention 2nm(3d + 2dv) per head (10nmd when
d = dv), halved for causal.

Prints one JSON line.  Options: --steps K --warmup W --gpus N (N must be 1)
--workload NAME --no-cpu-baseline --cpu-heads H --no-proj.

Beside the backward, "layer_proj" times the projection gradients of the
multi-head layer around it at the workload's sizes (T = B n tokens,
d_model = H d): attn_out_proj_bwd (dW_O, dO_cat) and attn_in_proj_bwd
(dW_Q, dW_K, dW_V, dX), 2 T d_model (2 H dv + 2 H d + H dv) x 2 flop, and
the same products through torch.matmul for context.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the dK/dV kernel (the dominant one) on causal_4k_d128, from
# rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the
# same counters read for a plain 1 GiB device copy (x2.0 and x1.0).  They
# hold only for the kernel sources they were taken on, identified by hash;
# after any change to those sources the traffic is reported as null.
KERNEL_SOURCES = ("attn_bwd_mfma.hip", "attn_bwd_dq_mfma.hip", "attn_device.h", "attn_launch.h")
MEASURED_TRAFFIC = {
    "workload": "causal_4k_d128",
    "sources_sha256": "7c90c0964c97c6b56e87ff4d5dbbd003c3ec7c4e1d43dd39522444875db6bdac",
    "bytes": {"bwd_dkdv": 7.6320e+08},
}


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "transformer_attn_bwd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    m = MEASURED_TRAFFIC
    if m["workload"] != workload or m["sources_sha256"] != kernel_sources_sha256():
        return None
    return m["bytes"].get(kernel)


def bwd_flops(w) -> float:
    f = 2.0 * w.n * w.m * (3 * w.d + 2 * w.dv) * w.B * w.H
    return f / 2 if w.causal else f


def fwd_flops(w) -> float:
    f = 2.0 * w.n * w.m * (w.d + w.dv) * w.B * w.H
    return f / 2 if w.causal else f


def dkdv_flops(w) -> float:
    # S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q
    f = 2.0 * w.n * w.m * (2 * w.d + 2 * w.dv) * w.B * w.H
    return f / 2 if w.causal else f


def dq_flops(w) -> float:
    # S, dP recomputed, dQ += dS K
    f = 2.0 * w.n * w.m * (2 * w.d + w.dv) * w.B * w.H
    return f / 2 if w.causal else f


def bwd_bytes(w) -> float:
    """Algorithmic HBM bytes of one backward: read Q,K,V,O,dO (bf16) and
    LSE; write dQ,dK,dV (bf16); D and rescaled LSE written and read once."""
    e = 2
    heads = w.B * w.H
    qk = heads * (w.n * w.d + w.m * w.d) * e
    vo = heads * (w.m * w.dv + 2 * w.n * w.dv) * e
    grads = heads * (w.n * w.d + w.m * w.d + w.m * w.dv) * e
    rows = heads * w.n * 4 * (1 + 2 * 2)
    return float(qk + vo + grads + rows)


def time_loop(fn, steps, torch, warmup=0):
    for _ in range(warmup):
        fn()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def step_times(fn, steps, torch):
    """Per-step durations (ms) from an event pair around each step."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)


def proj_flops(T, dm, hd, hdv) -> float:
    # dW_O and dO_cat: 2 T dm hdv each; dW_Q, dW_K, dW_V: 2 T dm (2 hd + hdv);
    # dX: 2 T dm (2 hd + hdv)
    return 2.0 * T * dm * (2 * hdv + 2 * (2 * hd + hdv))


def proj_bench(w, steps, torch, attn):
    """Projection gradients at the workload's layer sizes (synthetic
    16-bit inputs on the GPU)."""
    T, hd, hdv = w.B * w.n, w.H * w.d, w.H * w.dv
    dm = hd
    dev = "cuda:0"
    dt = w.torch_dtype
    g = torch.Generator(device=dev).manual_seed(9)
    r = lambda *shape: torch.randn(shape, generator=g, device=dev).to(dt)
    X, G, o_cat = r(T, dm), r(T, dm), r(T, hdv)
    Wq, Wk, Wv, Wo = r(dm, hd), r(dm, hd), r(dm, hdv), r(hdv, dm)
    dQ, dK, dV = r(T, hd), r(T, hd), r(T, hdv)
    dw_o, do_cat = attn.out_proj_bwd(o_cat, G, Wo)
    grads = attn.in_proj_bwd(X, Wq, Wk, Wv, dQ, dK, dV)
    out_ms = time_loop(lambda: attn.out_proj_bwd(o_cat, G, Wo, dw_o=dw_o, do_cat=do_cat),
                       steps, torch, 3)
    in_ms = time_loop(lambda: attn.in_proj_bwd(X, Wq, Wk, Wv, dQ, dK, dV, out=grads),
                      steps, torch, 3)

    def torch_products():
        torch.matmul(o_cat.t(), G)
        torch.matmul(G, Wo.t())
        for dP in (dQ, dK, dV):
            torch.matmul(X.t(), dP)
        torch.matmul(dQ, Wq.t()).add_(torch.matmul(dK, Wk.t())).add_(torch.matmul(dV, Wv.t()))

    ref_ms = time_loop(torch_products, steps, torch, 3)
    f = proj_flops(T, dm, hd, hdv)
    ms = out_ms + in_ms
    return {
        "T": T, "d_model": dm, "hd": hd, "hdv": hdv, "flops": f,
        "out_proj_ms": round(out_ms, 4), "in_proj_ms": round(in_ms, 4),
        "tflops": round(f / (ms * 1e-3) / 1e12, 2),
        "pct_of_peak": round(100.0 * f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "torch_matmul_ms": round(ref_ms, 4),
    }


def cpu_baseline(w, inputs, heads_wanted):
    """The float64 oracle's backward on a bounded sample of the workload's
    heads, on the host cores; reported in the metric's unit."""
    import numpy as np
    import oracle
    threads = oracle.num_threads()
    # about 20 s of float64 work at the headline size: four heads per thread
    nh = max(1, min(heads_wanted or 4 * threads, w.B * w.H))
    q, k, v, do = (t.reshape(w.B * w.H, *t.shape[2:])[:nh].double().numpy() for t in inputs)
    q, k, v, do = (np.ascontiguousarray(x[None]) for x in (q, k, v, do))
    t0 = time.perf_counter()
    oracle.attn_bwd(q, k, v, do, scale=w.softmax_scale, causal=w.causal)
    dt = time.perf_counter() - t0
    per_head = bwd_flops(w) / (w.B * w.H)
    return {
        "value": per_head * nh / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{nh} of {w.B * w.H} heads of {w.name} (float64 backward incl. recomputing "
                  f"P, O, D), {dt:.1f} s wall on {threads} OpenMP threads",
        "seconds": dt, "heads": nh,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0)
    ap.add_argument("--no-proj", action="store_true", help="skip the projection-gradient timing")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size first (a known-traffic "
                         "reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each "
              "(batch, head) is independent, so several GPUs would split the heads)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attn_bwd_amd as attn
    from transformer_attn_bwd_amd.workloads import HEADLINE, WORKLOADS, make_inputs

    w = WORKLOADS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: {w.describe()}", file=sys.stderr, flush=True)

    if args.copy_probe_mib > 0:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    inputs_cpu = make_inputs(w, "cpu")
    q, k, v, do = (t.to(dev) for t in inputs_cpu)
    o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal)
    ws = torch.empty(max(attn.bwd_workspace_bytes(w.B, w.H, w.n, w.m, w.d, w.dv, q.dtype), 1),
                     dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def bwd_step(stages=None):
        attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal, workspace=ws,
                 dq=dq, dk=dk, dv=dv, stages=stages)

    def fwd_step():
        attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal, out=o, lse=lse)

    for _ in range(args.warmup):
        fwd_step()
        bwd_step()
    torch.cuda.synchronize()
    print("bench: warmup done", file=sys.stderr, flush=True)

    # timed region: K backward steps, bracketed by device synchronisation
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms = time_loop(bwd_step, args.steps, torch)
    t_wall = time.perf_counter() - t_wall
    print(f"bench: {args.steps} steps, {ms:.3f} ms/step", file=sys.stderr, flush=True)
    ok = bool(torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all())
    # the spread of single steps (L2 not flushed between steps)
    per_step = step_times(bwd_step, args.steps, torch)

    # per-kernel average launch durations (HIP events on the launch stream)
    kern_ms = {
        "preprocess": time_loop(lambda: bwd_step(["preprocess"]), args.steps, torch, 3),
        "dkdv": time_loop(lambda: bwd_step(["dkdv"]), args.steps, torch, 3),
        "dq": time_loop(lambda: bwd_step(["dq"]), args.steps, torch, 3),
        # what a whole 16-bit backward launches first: the dQ pass with the
        # preprocess in its prologue
        "dq_with_preprocess": time_loop(lambda: bwd_step(["preprocess", "dq"]), args.steps,
                                        torch, 3),
    }
    fwd_ms = time_loop(fwd_step, args.steps, torch, 3)
    # restore outputs of a whole backward after the single-stage runs
    bwd_step()
    torch.cuda.synchronize()

    flops = bwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    dk_tf = dkdv_flops(w) / (kern_ms["dkdv"] * 1e-3) / 1e12
    dominant = max(("dkdv", "dq"), key=lambda kname: kern_ms[kname])
    dom_flops = dkdv_flops(w) if dominant == "dkdv" else dq_flops(w)
    dom_tf = dom_flops / (kern_ms[dominant] * 1e-3) / 1e12

    result = {
        "metric": "attn backward TFLOP/s (bf16, causal, d=128, N=4096) + % of MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp16": "f16", "fp32": "f32"}[w.dtype],
        "data": "synthetic (seeded N(0,1) inputs, see transformer_attn_bwd_amd/workloads.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "m": w.m, "d": w.d,
                   "dv": w.dv, "causal": w.causal, "seed": w.seed, "scale": w.softmax_scale,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": flops,
        "kernels_ms": {k_: round(v_, 4) for k_, v_ in kern_ms.items()},
        "fwd": {"ms": round(fwd_ms, 4),
                "tflops": round(fwd_flops(w) / (fwd_ms * 1e-3) / 1e12, 2),
                "pct_of_peak": round(100.0 * fwd_flops(w) / (fwd_ms * 1e-3) / 1e12
                                     / PEAK_BF16_TFLOPS, 2)},
        "roofline": {
            "kernel": f"bwd_{dominant}",
            "bound": "mfma",
            "achieved": round(dom_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name, f"bwd_{dominant}"),
        },
        "dkdv_tflops": round(dk_tf, 2),
        "hbm_algorithmic_GBps": round(bwd_bytes(w) / (ms * 1e-3) / 1e9, 1),
        "outputs_finite": ok,
        "wall_s_timed": round(t_wall, 3),
    }
    if not args.no_proj and w.dtype != "fp32":
        print("bench: projection gradients ...", file=sys.stderr, flush=True)
        result["layer_proj"] = proj_bench(w, max(5, args.steps // 2), torch, attn)
    if not args.no_cpu_baseline and w.dtype != "fp32":
        print("bench: cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inputs_cpu, args.cpu_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

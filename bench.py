#!/usr/bin/env python3
"""Throughput of the attention backward on one MI355X.

Workload: causal, bf16, B=2, H=32, n=m=4096, d=dv=128, seed 2, scale
1/sqrt(128).  A step is one backward pass (D preprocess, dK/dV kernel, dQ
kernel) over inputs already resident in HBM; O and LSE come from the
forward kernel, which runs before the timed region and is timed on its own
as context.  FLOPs follow the convention 2nm(3d + 2dv) per head (10nmd when
d = dv), halved for causal.

Before the W warmup steps, untimed backward steps run for SETTLE_S seconds
so that the GPU clock has settled under sustained load (it ramps for tens of
milliseconds after idle); the JSON line's "settle" field reports them.
Single-step durations come from HIP events without the system-scope fence
(a default event writes back and invalidates the caches between steps).

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
PEAK_F32_TFLOPS = 157.3     # MI355X float32 vector peak (the float32 path runs on VALU)
SETTLE_S = 0.25             # seconds of back-to-back backward steps before any timing


def peak_tflops(w) -> float:
    return PEAK_F32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS

# HBM bytes per launch of the dK/dV kernel (the dominant one) on causal_4k_d128, from
# rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the
# same counters read for a plain 1 GiB device copy (x2.0 and x1.0).  They
# hold only for the kernel sources they were taken on, identified by hash;
# after any change to those sources the traffic is reported as null.
KERNEL_SOURCES = ("attn_bwd_mfma.hip", "attn_bwd_dkdv.h", "attn_bwd_dq_mfma.hip", "attn_device.h",
                  "attn_launch.h", "attn_bwd_dkdv_dss.hip", "attn_bwd_dq_ds.hip")
MEASURED_TRAFFIC = {
    "workload": "causal_4k_d128",
    "sources_sha256": "ecdfe459ee4e70701903f2e95d83000f83945d4f61cdae6ed5e74e1b09fca7af",
    "bytes": {"bwd_dkdv": 7.6447e+08},
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


def dq_ds_flops(w) -> float:
    # dQ += dS K from the stored dS: the one product of the five left to it
    f = 2.0 * w.n * w.m * w.d * w.B * w.H
    return f / 2 if w.causal else f


def ds_tile_bytes(w) -> float:
    """Bytes of the stored-dS mode's dS tiles (16-bit, 256 x 256 each: the
    diagonal and lower tiles under the causal mask, all without it)."""
    nb, mb = -(-w.n // 256), -(-w.m // 256)
    tiles = nb * (nb + 1) // 2 if w.causal else nb * mb
    return float(w.B * w.H * tiles * 256 * 256 * 2)


def dq_ds_bytes(w) -> float:
    """Algorithmic HBM bytes of the dQ-from-dS pass: read the dS tiles and K
    (16-bit); write dQ (16-bit)."""
    return ds_tile_bytes(w) + float(w.B * w.H * (w.m * w.d + w.n * w.d) * 2)


def mode_kernels(w, mode):
    """(FLOPs, algorithmic bytes) of the dK/dV and dQ kernels in a dQ mode
    (the atomic mode's are set by its split, in mode_figures)."""
    if mode == "stored_ds":
        return {"dkdv": (dkdv_flops(w), dkdv_bytes(w) + ds_tile_bytes(w)),
                "dq": (dq_ds_flops(w), dq_ds_bytes(w))}
    return {"dkdv": (dkdv_flops(w), dkdv_bytes(w)), "dq": (dq_flops(w), dq_bytes(w))}


def resolved_mode(attn, w, torch_dtype) -> str:
    """The dQ mode the library's ATTN_DQ_AUTO takes for a workload: read off
    its workspace size, which is that of the mode it picks."""
    def size(mode):
        return attn.bwd_workspace_bytes(w.B, w.H, w.n, w.m, w.d, w.dv, torch_dtype,
                                        dq_mode=mode, causal=w.causal)
    auto = size("auto")
    if auto == size("stored_ds") and auto != size("separate"):
        return "stored_ds"
    return "separate"


def dkdv_bytes(w) -> float:
    """Algorithmic HBM bytes of the dK/dV kernel: read Q, K, V, dO (16-bit),
    LSE2 and D (float32); write dK and dV (16-bit)."""
    e = 2
    heads = w.B * w.H
    reads = heads * (w.n * w.d + w.m * w.d + w.m * w.dv + w.n * w.dv) * e + heads * w.n * 8
    writes = heads * (w.m * w.d + w.m * w.dv) * e
    return float(reads + writes)


def dq_bytes(w) -> float:
    """Algorithmic HBM bytes of the dQ pass with its preprocess prologue:
    read Q, K, V, O, dO (16-bit) and LSE (float32); write dQ (16-bit) and
    LSE2 and D (float32)."""
    e = 2
    heads = w.B * w.H
    reads = heads * (w.n * w.d + w.m * w.d + w.m * w.dv + 2 * w.n * w.dv) * e + heads * w.n * 4
    writes = heads * w.n * w.d * e + heads * w.n * 8
    return float(reads + writes)


def roofline_bound(flops: float, nbytes: float) -> str:
    """"mfma" when the kernel's arithmetic intensity (flop per algorithmic
    HBM byte) is above the machine balance of dense bf16 MFMA over HBM
    (2516.6 TFLOP/s / 8 TB/s = 315 flop/B), else "hbm"."""
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    return "mfma" if flops / nbytes > ridge else "hbm"


def pairs_from(w, key0: int) -> float:
    """Visible (query, key) pairs with key index >= key0, over all heads."""
    key0 = min(max(key0, 0), w.m)
    if w.causal:
        cnt = sum(max(0, w.n - j) for j in range(key0, w.m))
    else:
        cnt = w.n * (w.m - key0)
    return float(cnt) * w.B * w.H


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


class _FenceFreeEvents:
    """HIP timing events created with hipEventDisableSystemFence, recorded on
    torch's current stream (the one the library launches on).  A default
    event ends in a system-scope release: a writeback and invalidation of
    the caches, which slows the step after it, so events between single
    steps would time a step that no back-to-back loop runs.  These events
    only timestamp; elapsed times are read after a device synchronisation."""
    FLAG = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self, torch):
        import ctypes
        # the HIP runtime torch already loaded (one copy per process)
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        self.ct = ctypes
        self.torch = torch

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.FLAG) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def record(self, ev):
        stream = self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def step_times(fn, steps, torch):
    """Per-step durations (ms) from a fence-free event pair around each of
    `steps` back-to-back steps, sorted (torch's events if the HIP runtime's
    symbols cannot be reached)."""
    try:
        ev = _FenceFreeEvents(torch)
    except OSError:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        ev.record(a)
        fn()
        ev.record(b)
    torch.cuda.synchronize()
    out = sorted(ev.elapsed_ms(a, b) for a, b in pairs)
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    return out


def settle(fn, torch, seconds):
    """Run fn back to back until the GPU has been busy for `seconds` and
    return (steps, seconds).  Under a sustained load the MI355X clock ramps
    for the first few tens of milliseconds (4k backward in groups of ten
    steps from idle: 1.14, 0.92, 0.88, 0.86, then 0.85 ms per step), so a
    throughput taken right after idle times the ramp, not the kernels."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return n, dt


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


# the other workloads timed beside the headline, in both dQ modes
TABLE_WORKLOADS = ("head_64_fp32", "causal_1k_d64", "causal_4k_d128", "causal_16k_d128",
                   "cross_512x2048_d128_dv64", "causal_4k_d128_fp16")


def mode_figures(w, run, steps, torch, split=None, mode="separate"):
    """Whole-backward and per-kernel timings of one dQ mode."""
    # the first launches after another workload's run come at a lower clock
    settle(run, torch, SETTLE_S)
    ms = time_loop(run, steps, torch, 2)
    med = step_times(run, steps, torch)[steps // 2]
    k_dkdv = time_loop(lambda: run(["dkdv"]), steps, torch, 2)
    k_dq = time_loop(lambda: run(["preprocess", "dq"]), steps, torch, 2)
    nkeys = (split or 0) * 256
    if split is None:
        kf = mode_kernels(w, mode)
        f_dkdv, f_dq = kf["dkdv"][0], kf["dq"][0]
    else:
        # the fused kernel also forms dS K for the keys past the split; the
        # separate pass recomputes S and dP only for the keys before it
        frac_sep = 1.0 - pairs_from(w, nkeys) / pairs_from(w, 0)
        f_dkdv = dkdv_flops(w) + 2.0 * w.d * pairs_from(w, nkeys)
        f_dq = dq_flops(w) * frac_sep
    kern = {"dkdv": (k_dkdv, f_dkdv), "dq": (k_dq, f_dq)}
    dom = max(kern, key=lambda k_: kern[k_][0])
    tf = bwd_flops(w) / (ms * 1e-3) / 1e12
    peak = peak_tflops(w)
    out = {
        "ms_mean": round(ms, 4), "ms_median": round(med, 4), "tflops": round(tf, 2),
        "pct_of_peak": round(100.0 * tf / peak, 2), "peak_tflops": peak,
        "kernels_ms": {"dkdv": round(k_dkdv, 4), "dq_with_preprocess": round(k_dq, 4)},
        "dominant": dom,
        "dominant_share_of_step": round(kern[dom][0] / ms, 3),
        "dominant_frac_of_peak": round(kern[dom][1] / (kern[dom][0] * 1e-3) / 1e12 / peak, 4),
    }
    if split is not None:
        out["split"] = split
    return out


def workload_table(names, steps, torch, attn, make_inputs, workloads):
    """For each workload: the backward in the separate-pass and stored-dS dQ
    modes, and in the atomic mode at the best of a few splits (leading
    256-key blocks left to the separate pass); the float32 workload in the
    separate pass only (the other modes are 16-bit), against the float32
    vector peak."""
    table = {}
    dev = "cuda:0"
    for name in names:
        w = workloads[name]
        print(f"bench: table {name} ...", file=sys.stderr, flush=True)
        q, k, v, do = (t.to(dev) for t in make_inputs(w, "cpu"))
        o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        wss = {}

        def runner(mode, split):
            key = mode
            if key not in wss:
                wss[key] = torch.empty(max(attn.bwd_workspace_bytes(
                    w.B, w.H, w.n, w.m, w.d, w.dv, q.dtype, dq_mode=mode, causal=w.causal), 1),
                    dtype=torch.uint8, device=dev)
            return lambda stages=None: attn.bwd(
                q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal, dq_mode=mode,
                dq_split=split, workspace=wss[key], dq=dq, dk=dk, dv=dv, stages=stages)

        row = {"flops": bwd_flops(w), "auto_mode": resolved_mode(attn, w, q.dtype),
               "separate": mode_figures(w, runner("separate", None), steps, torch)}
        if w.dtype == "fp32":
            table[name] = row
            continue
        row["stored_ds"] = mode_figures(w, runner("stored_ds", None), steps, torch,
                                        mode="stored_ds")
        nkb = (w.m + 255) // 256
        splits = sorted({0} | {max(1, (nkb * f) // 8) for f in (1, 2, 3, 4, 6)})
        tried = {sp: time_loop(runner("atomic", sp), max(3, steps // 2), torch, 2)
                 for sp in splits}
        best = min(tried, key=tried.get)
        row["atomic"] = mode_figures(w, runner("atomic", best), steps, torch, best)
        row["atomic"]["splits_ms"] = {str(sp): round(t, 4) for sp, t in tried.items()}
        table[name] = row
        del q, k, v, do, o, lse, dq, dk, dv, wss
        torch.cuda.empty_cache()
    return table


def cpu_baseline(w, inputs, heads_wanted):
    """The float64 oracle's backward on a bounded sample of the workload's
    heads, on the host cores; reported in the metric's unit."""
    import numpy as np
    import oracle
    threads = oracle.num_threads()
    affinity = len(os.sched_getaffinity(0))
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
        "seconds": dt, "heads": nh, "omp_threads": threads, "affinity_cpus": affinity,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dq-mode", default="auto", choices=("auto", "separate", "stored_ds"),
                    help="dQ mode of the headline line (default: the library's own choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0)
    ap.add_argument("--no-proj", action="store_true", help="skip the projection-gradient timing")
    ap.add_argument("--no-table", action="store_true",
                    help="skip the other workloads and the atomic dQ mode")
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
    # the library's own choice of dQ mode (ATTN_DQ_AUTO) is what is timed,
    # unless --dq-mode names another (for profiling the other modes)
    mode = resolved_mode(attn, w, q.dtype) if args.dq_mode == "auto" else args.dq_mode
    ws = torch.empty(max(attn.bwd_workspace_bytes(w.B, w.H, w.n, w.m, w.d, w.dv, q.dtype,
                                                  dq_mode=args.dq_mode, causal=w.causal), 1),
                     dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def bwd_step(stages=None):
        attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal, workspace=ws,
                 dq=dq, dk=dk, dv=dv, stages=stages, dq_mode=args.dq_mode)

    def fwd_step():
        attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal, out=o, lse=lse)

    # the clock settles under sustained load first (see settle()), then the
    # W warmup steps
    settle_steps, settle_s = settle(bwd_step, torch, SETTLE_S)
    for _ in range(args.warmup):
        fwd_step()
        bwd_step()
    torch.cuda.synchronize()
    print(f"bench: clock settled ({settle_steps} steps, {settle_s:.2f} s), warmup done",
          file=sys.stderr, flush=True)

    # timed region: K backward steps, bracketed by device synchronisation
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms = time_loop(bwd_step, args.steps, torch)
    t_wall = time.perf_counter() - t_wall
    # the spread of single steps (L2 not flushed between steps), right after
    # the timed loop: an idle gap (a host synchronisation) lowers the clock
    per_step = step_times(bwd_step, args.steps, torch)
    print(f"bench: {args.steps} steps, {ms:.3f} ms/step", file=sys.stderr, flush=True)
    ok = bool(torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all())

    # per-kernel average launch durations (HIP events on the launch stream),
    # on a settled clock again after the host synchronisation above
    settle(bwd_step, torch, SETTLE_S)
    kern_ms = {
        "preprocess": time_loop(lambda: bwd_step(["preprocess"]), args.steps, torch, 3),
        "dkdv": time_loop(lambda: bwd_step(["dkdv"]), args.steps, torch, 3),
        "dq": time_loop(lambda: bwd_step(["dq"]), args.steps, torch, 3),
        # the separate mode launches the dQ pass first with the preprocess in
        # its prologue; the stored-dS mode launches the two on their own
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
    dom_flops, dom_bytes = mode_kernels(w, mode)[dominant]
    dom_tf = dom_flops / (kern_ms[dominant] * 1e-3) / 1e12
    mask = "causal" if w.causal else "non-causal"
    shape = f"N={w.n}" if w.n == w.m else f"n={w.n}, m={w.m}"
    dims = f"d={w.d}" if w.d == w.dv else f"d={w.d}, dv={w.dv}"

    result = {
        "metric": f"attn backward TFLOP/s ({w.dtype}, {mask}, {dims}, {shape}) + % of "
                  + ("float32 vector peak" if w.dtype == "fp32" else "MFMA peak"),
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
        "pct_of_peak": round(100.0 * tflops / peak_tflops(w), 2),
        "flops_per_step": flops,
        "dq_mode": mode,
        "kernels_ms": {k_: round(v_, 4) for k_, v_ in kern_ms.items()},
        "fwd": {"ms": round(fwd_ms, 4),
                "tflops": round(fwd_flops(w) / (fwd_ms * 1e-3) / 1e12, 2),
                "pct_of_peak": round(100.0 * fwd_flops(w) / (fwd_ms * 1e-3) / 1e12
                                     / peak_tflops(w), 2)},
        "roofline": {
            "kernel": f"bwd_{dominant}",
            # the float32 path runs on the vector ALUs, not the matrix cores
            "bound": "alu" if w.dtype == "fp32" else roofline_bound(dom_flops, dom_bytes),
            "achieved": round(dom_tf, 2),
            "peak": peak_tflops(w),
            "unit": "TFLOP/s",
            "frac": round(dom_tf / peak_tflops(w), 4),
            # stored for the default mode's kernels only
            "traffic": (measured_traffic(w.name, f"bwd_{dominant}") if mode == "separate"
                        else None),
            "algorithmic_bytes": dom_bytes,
        },
        "dkdv_tflops": round(dk_tf, 2),
        "hbm_algorithmic_GBps": round(bwd_bytes(w) / (ms * 1e-3) / 1e9, 1),
        "settle": {"steps": settle_steps, "seconds": round(settle_s, 3),
                   "note": "untimed backward steps run until the GPU clock settles, "
                           "before the warmup steps"},
        "outputs_finite": ok,
        "wall_s_timed": round(t_wall, 3),
    }
    if not args.no_table:
        result["workloads"] = workload_table(
            [x for x in TABLE_WORKLOADS], max(5, args.steps // 2), torch, attn, make_inputs,
            WORKLOADS)
    if not args.no_proj and w.dtype != "fp32":
        print("bench: projection gradients ...", file=sys.stderr, flush=True)
        result["layer_proj"] = proj_bench(w, max(5, args.steps // 2), torch, attn)
    if not args.no_cpu_baseline and w.dtype != "fp32":
        print("bench: cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inputs_cpu, args.cpu_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Helpers shared by the GPU tests: running the library on a workload and
comparing with the oracle.  Test infrastructure; not imported by the product."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd.workloads import Workload, make_inputs

# Tolerances: bf16 path max|err| / max|ref| <= 2e-2 per output tensor; the
# fp32 path 1e-5 in the same per-tensor relative form (LSE absolute).  The
# float16 path rounds P, dS and the outputs with a unit roundoff of 2^-11
# instead of bfloat16's 2^-8, so its bar is the bf16 one scaled by 2^-3.
TOL = {"bf16": 2e-2, "fp16": 2.5e-3, "fp32": 1e-5}
LSE_TOL = {"bf16": 1e-3, "fp16": 1e-3, "fp32": 1e-5}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.max(np.abs(ref)))
    if denom == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / denom)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def run_gpu(w: Workload, inputs=None, dev="cuda:0"):
    """Forward then backward on the GPU; returns dict of device tensors."""
    q, k, v, do = inputs if inputs is not None else make_inputs(w, dev)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal)
    torch.cuda.synchronize()
    return {"q": q, "k": k, "v": v, "do": do, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def oracle_full(w: Workload, inputs):
    q, k, v, do = (to64(t) for t in inputs)
    return oracle.attn_bwd(q, k, v, do, scale=w.softmax_scale, causal=w.causal)


def compare_full(w: Workload, gpu: dict, ref: dict, tol=None, lse_tol=None) -> dict:
    tol = TOL[w.dtype] if tol is None else tol
    lse_tol = LSE_TOL[w.dtype] if lse_tol is None else lse_tol
    errs = {}
    for name in ("o", "dq", "dk", "dv"):
        errs[name] = rel_err(to64(gpu[name]), ref[name])
    errs["lse_abs"] = float(np.max(np.abs(to64(gpu["lse"]) - ref["lse"]))) if ref["lse"].size else 0.0
    say(f"  errors {w.name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for name in ("o", "dq", "dk", "dv"):
        assert errs[name] <= tol, (w.name, name, errs[name])
    assert errs["lse_abs"] <= lse_tol, (w.name, "lse", errs["lse_abs"])
    return errs

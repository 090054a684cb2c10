"""Whole-tensor parity at the full workload sizes, in the launch
configuration the benchmark times: every element of O, LSE, dQ, dK and dV
against the float64 oracle, with the per-tensor bar max|err| / max|ref|
taken over the whole tensor.

Every head of the 1k/d64, 4k/d128 (bf16 and fp16) and 512x2048 cross
workloads is compared; the 16k/d128 workload is compared on two whole heads
(the oracle needs about 4 s per head of it on 16 cores) and by sampled rows
elsewhere.  The backward runs in every dQ mode on the same forward: the
separate pass (what ATTN_DQ_AUTO picks), the atomic mode at a middle split
and the stored-dS mode.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd.workloads import WORKLOADS, make_inputs

from gpu_util import LSE_TOL, TOL, rel_err, say, to64

pytestmark = pytest.mark.gpu

WHOLE = ["causal_1k_d64", "causal_4k_d128", "causal_4k_d128_fp16", "cross_512x2048_d128_dv64"]


def _forward_backward(w, inputs, modes):
    q, k, v, do = (t.to("cuda:0") for t in inputs)
    o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal)
    grads = {}
    for mode, split in modes:
        grads[(mode, split)] = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale,
                                        causal=w.causal, dq_mode=mode, dq_split=split)
    torch.cuda.synchronize()
    return o, lse, grads


def _modes(w):
    nkb = (w.m + 255) // 256
    return [("separate", None), ("atomic", nkb // 2), ("stored_ds", None)]


def _check(w, got_o, got_lse, grads, ref, label):
    tol = TOL[w.dtype]
    errs = {"o": rel_err(to64(got_o), ref["o"]),
            "lse_abs": float(np.max(np.abs(to64(got_lse) - ref["lse"])))}
    say(f"  {label}: o={errs['o']:.3e} lse_abs={errs['lse_abs']:.3e}")
    assert errs["o"] <= tol, (label, "o", errs["o"])
    assert errs["lse_abs"] <= LSE_TOL[w.dtype], (label, "lse", errs["lse_abs"])
    for key, (dq, dk, dv) in grads.items():
        e = {"dq": rel_err(to64(dq), ref["dq"]), "dk": rel_err(to64(dk), ref["dk"]),
             "dv": rel_err(to64(dv), ref["dv"])}
        say(f"  {label} {key}: " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in e.items()))
        for name, val in e.items():
            assert val <= tol, (label, key, name, val)


@pytest.mark.parametrize("name", WHOLE)
def test_whole_tensors_every_head(name):
    w = WORKLOADS[name]
    say(f"case whole {w.describe()}")
    inputs = make_inputs(w)
    o, lse, grads = _forward_backward(w, inputs, _modes(w))
    ref = oracle.attn_bwd(*(to64(t) for t in inputs), scale=w.softmax_scale, causal=w.causal)
    _check(w, o, lse, grads, ref, name)


def test_causal_16k_two_whole_heads():
    """Heads (0, 0) and (0, H-1) of the B=1, H=32, n=m=16384, d=128 causal
    workload, every element, from one launch over all 32 heads."""
    w = WORKLOADS["causal_16k_d128"]
    say(f"case two whole heads {w.describe()}")
    inputs = make_inputs(w)
    o, lse, grads = _forward_backward(w, inputs, _modes(w))
    heads = [0, w.H - 1]
    sub = [to64(t[:, heads]) for t in inputs]
    ref = oracle.attn_bwd(*sub, scale=w.softmax_scale, causal=w.causal)
    picked = {key: tuple(g[:, heads] for g in gr) for key, gr in grads.items()}
    _check(w, o[:, heads], lse[:, heads], picked, ref, f"{w.name} heads {heads}")

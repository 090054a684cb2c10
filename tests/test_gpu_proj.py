"""GPU parity of the projection gradients around attention (eulerpad
"Attention backward" Problems 7 and 10; datatweets "Step 4") against the
oracle's float64 products, and of the whole layer backward chained through
the [B, seq, H, dim] layout:

    attn_out_proj_bwd -> dO -> attn_bwd_ex (bshd) -> dQ, dK, dV -> attn_in_proj_bwd

Bars (max|err| / max|ref| per tensor): float32 weight gradients 1e-5 (the
inputs are exact in both; only the float32 accumulation order differs);
16-bit outputs twice their unit roundoff, 4e-3 (bf16) and 1e-3 (fp16), for
the single rounding of the result; the chained layer, whose intermediate
tensors are rounded to 16 bits, the attention bar (2e-2 bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attn_bwd_amd as attn

from gpu_util import TOL, rel_err, say, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
OUT_TOL = {"bf16": 4e-3, "fp16": 1e-3}
W_TOL = 1e-5


def _rand(shape, g, scale=1.0, dtype="bf16"):
    return (torch.randn(shape, generator=g) * scale).to(DT[dtype])


@pytest.mark.parametrize("T,dm,hdv,dtype", [
    (600, 320, 256, "bf16"),     # ragged against the 256 x 256 tiles in every direction
    (257, 64, 96, "bf16"),
    (1024, 512, 512, "fp16"),
    (1, 8, 8, "bf16"),
    (0, 64, 64, "bf16"),         # no tokens: dW_O = 0
])
def test_out_proj_bwd(T, dm, hdv, dtype):
    say(f"case out_proj T={T} d_model={dm} hdv={hdv} {dtype}")
    g = torch.Generator().manual_seed(T + dm + hdv)
    o_cat, G, Wo = _rand((T, hdv), g, 1.0, dtype), _rand((T, dm), g, 1.0, dtype), \
        _rand((hdv, dm), g, 0.05, dtype)
    dw, do_cat = attn.out_proj_bwd(o_cat.cuda(), G.cuda(), Wo.cuda())
    torch.cuda.synchronize()
    ref = oracle.out_proj_bwd(o_cat, G, Wo)
    e_w = rel_err(to64(dw), ref["dw_o"]) if T else float(torch.count_nonzero(dw))
    e_o = rel_err(to64(do_cat), ref["do_cat"]) if T else 0.0
    say(f"  dw_o {e_w:.3e} do_cat {e_o:.3e}")
    assert dw.dtype == torch.float32 and do_cat.dtype == DT[dtype]
    assert e_w <= W_TOL and e_o <= OUT_TOL[dtype]


@pytest.mark.parametrize("T,dm,hd,hdv,dtype", [
    (600, 320, 256, 128, "bf16"),
    (333, 136, 72, 40, "bf16"),
    (1024, 256, 512, 512, "fp16"),
])
def test_in_proj_bwd(T, dm, hd, hdv, dtype):
    say(f"case in_proj T={T} d_model={dm} hd={hd} hdv={hdv} {dtype}")
    g = torch.Generator().manual_seed(T + dm + hd + hdv)
    X = _rand((T, dm), g, 1.0, dtype)
    Wq, Wk, Wv = _rand((dm, hd), g, 0.05, dtype), _rand((dm, hd), g, 0.05, dtype), \
        _rand((dm, hdv), g, 0.05, dtype)
    dQ, dK, dV = _rand((T, hd), g, 1.0, dtype), _rand((T, hd), g, 1.0, dtype), \
        _rand((T, hdv), g, 1.0, dtype)
    out = attn.in_proj_bwd(*(t.cuda() for t in (X, Wq, Wk, Wv, dQ, dK, dV)))
    torch.cuda.synchronize()
    ref = oracle.in_proj_bwd(X, Wq, Wk, Wv, dQ, dK, dV)
    errs = {k: rel_err(to64(out[k]), ref[k]) for k in ("dw_q", "dw_k", "dw_v", "dx")}
    say("  " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for k in ("dw_q", "dw_k", "dw_v"):
        assert out[k].dtype == torch.float32 and errs[k] <= W_TOL, (k, errs[k])
    assert errs["dx"] <= OUT_TOL[dtype]


def test_layer_backward_chain():
    """The whole layer: X -> (Q, K, V) -> causal attention per head -> O_cat
    -> Y = O_cat W_O, differentiated on the GPU through the library alone
    (tensors stay [T, H dim] = [B, n, H, dim]) and by the oracle's chain in
    float64 on the same 16-bit inputs."""
    B, n, H, d, dv, dm = 2, 300, 4, 64, 64, 320
    T = B * n
    g = torch.Generator().manual_seed(77)
    X = _rand((T, dm), g)
    Wq, Wk, Wv = (_rand((dm, H * w), g, dm ** -0.5) for w in (d, d, dv))
    Wo = _rand((H * dv, dm), g, (H * dv) ** -0.5)
    G = _rand((T, dm), g)
    # the projections themselves are the forward's business: done here in
    # float64 and rounded, as the layer's stored activations would be
    Q, K, V = ((X.double() @ W.double()).to(torch.bfloat16) for W in (Wq, Wk, Wv))
    dev = "cuda:0"
    q, k, v = (t.reshape(B, n, H, -1).to(dev) for t in (Q, K, V))
    o, lse = attn.fwd(q, k, v, mask="causal", layout="bshd")
    dw_o, do_cat = attn.out_proj_bwd(o.reshape(T, H * dv), G.to(dev), Wo.to(dev))
    dq, dk, dvv = attn.bwd(q, k, v, o, do_cat.reshape(B, n, H, dv), lse, mask="causal",
                           layout="bshd")
    grads = attn.in_proj_bwd(X.to(dev), Wq.to(dev), Wk.to(dev), Wv.to(dev),
                             dq.reshape(T, -1), dk.reshape(T, -1), dvv.reshape(T, -1))
    torch.cuda.synchronize()

    # oracle chain
    heads = lambda M, w: to64(M).reshape(B, n, H, w).transpose(0, 2, 1, 3)
    cat = lambda M: M.transpose(0, 2, 1, 3).reshape(T, -1)
    ro, _ = oracle.attn_fwd(heads(Q, d), heads(K, d), heads(V, dv), causal=True)
    a = oracle.out_proj_bwd(cat(ro), G, Wo)
    r = oracle.attn_bwd(heads(Q, d), heads(K, d), heads(V, dv),
                        a["do_cat"].reshape(B, n, H, dv).transpose(0, 2, 1, 3), causal=True)
    b = oracle.in_proj_bwd(X, Wq, Wk, Wv, cat(r["dq"]), cat(r["dk"]), cat(r["dv"]))
    errs = {
        "dw_o": rel_err(to64(dw_o), a["dw_o"]),
        "do": rel_err(to64(do_cat), a["do_cat"]),
        "dw_q": rel_err(to64(grads["dw_q"]), b["dw_q"]),
        "dw_k": rel_err(to64(grads["dw_k"]), b["dw_k"]),
        "dw_v": rel_err(to64(grads["dw_v"]), b["dw_v"]),
        "dx": rel_err(to64(grads["dx"]), b["dx"]),
    }
    say("  layer " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL["bf16"], (k_, v_)


def test_projection_sizes_sampled():
    """The headline layer's sizes (B=2, n=4096, H=32, d=128: T = 8192,
    d_model = 4096): sampled rows and columns of every output against the
    oracle's products restricted to them."""
    T, dm, hd = 8192, 4096, 4096
    g = torch.Generator().manual_seed(5)
    X, G = _rand((T, dm), g), _rand((T, dm), g)
    o_cat = _rand((T, hd), g)
    Wq, Wk, Wv = (_rand((dm, hd), g, dm ** -0.5) for _ in range(3))
    Wo = _rand((hd, dm), g, hd ** -0.5)
    dQ, dK, dV = (_rand((T, hd), g) for _ in range(3))
    dev = "cuda:0"
    dw_o, do_cat = attn.out_proj_bwd(o_cat.to(dev), G.to(dev), Wo.to(dev))
    pr = attn.in_proj_bwd(*(t.to(dev) for t in (X, Wq, Wk, Wv, dQ, dK, dV)))
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows_t = np.sort(rng.choice(T, 24, replace=False))
    rows_w = np.sort(rng.choice(dm, 24, replace=False))
    rows_h = np.sort(rng.choice(hd, 24, replace=False))
    x64, g64, o64 = to64(X), to64(G), to64(o_cat)
    checks = {
        "dw_o": (to64(dw_o[rows_h]), o64[:, rows_h].T @ g64, W_TOL),
        "do_cat": (to64(do_cat[rows_t]), g64[rows_t] @ to64(Wo).T, OUT_TOL["bf16"]),
        "dw_q": (to64(pr["dw_q"][rows_w]), x64[:, rows_w].T @ to64(dQ), W_TOL),
        "dw_k": (to64(pr["dw_k"][rows_w]), x64[:, rows_w].T @ to64(dK), W_TOL),
        "dw_v":(to64(pr["dw_v"][rows_w]), x64[:, rows_w].T @ to64(dV), W_TOL),
        "dx": (to64(pr["dx"][rows_t]),
               sum(to64(dP[rows_t]) @ to64(W).T for dP, W in ((dQ, Wq), (dK, Wk), (dV, Wv))),
               OUT_TOL["bf16"]),
    }
    for name, (got, ref, tol) in checks.items():
        e = rel_err(got, ref)
        say(f"  {name} {e:.3e}")
        assert e <= tol, (name, e)

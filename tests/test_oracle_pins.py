"""Pins of the float64 oracle to what the pages and the mathematics fix.

None of these compares the oracle with a copy of its own formula: each check
is a printed value, a closed form, an invariant, a finite difference or a
library routine (torch autograd, scipy's softmax) that reaches the same
gradient by a different road.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- printed values

def test_uniform_forward_example():
    """mlgrind 'Examples': Q = K = 0 gives uniform P and Out = mean of V's rows."""
    g = _golden("mlgrind_uniform_examples.json")["forward"]
    o, _ = oracle.attn_fwd(np.array(g["Q"]), np.array(g["K"]), np.array(g["V"]), causal=g["causal"])
    np.testing.assert_allclose(o, np.array(g["Out"]), rtol=0, atol=1e-14)


def test_uniform_backward_example():
    """mlgrind 'Examples': dV = P^T dOut with P = 1/3 prints 0.6667 everywhere."""
    gj = _golden("mlgrind_uniform_examples.json")
    f, b = gj["forward"], gj["backward"]
    r = oracle.attn_bwd(np.array(f["Q"]), np.array(f["K"]), np.array(f["V"]), np.array(b["dOut"]))
    half_ulp = 0.5 * 10.0 ** (-b["printed_decimals"])
    assert np.all(np.abs(r["dv"] - np.array(b["dV_printed"])) <= half_ulp)
    np.testing.assert_allclose(r["dv"], np.full((3, 2), 2.0 / 3.0), rtol=0, atol=1e-15)
    # K = 0 makes dQ = s dS K vanish and Q = 0 makes dK = s dS^T Q vanish
    # (eulerpad Problems 5 and 6), exactly.
    assert np.all(r["dq"] == 0.0) and np.all(r["dk"] == 0.0)


def _toy_head():
    """The datatweets toy head, drawn as its 'Setup' section describes."""
    rec = _golden("datatweets_toy_head.json")["recipe"]
    rs = np.random.RandomState(rec["seed"])
    t = {}
    for name in rec["draw_order"]:
        t[name] = rs.randn(*rec["shapes"][name]) * rec["multipliers"][name]
    return t


def _toy_loss(X, Wq, Wk, Wv, G):
    # projections are test-side glue; the attention itself is the oracle's
    o, _ = oracle.attn_fwd(X @ Wq, X @ Wk, X @ Wv, scale=1.0 / np.sqrt(Wq.shape[1]))
    return float(np.sum(o * G))


def test_toy_head_printed_loss():
    """datatweets 'A Scalar Loss So dout Is Known' prints L = -0.292686."""
    pr = _golden("datatweets_toy_head.json")["printed"]
    t = _toy_head()
    L = _toy_loss(t["X"], t["Wq"], t["Wk"], t["Wv"], t["G"])
    assert round(L, pr["L_decimals"]) == pr["L"]


def _max_rel_err(a, n):
    # datatweets 'Proving It': max |a - n| / max(|a|, |n|), 1e-12 in the denominator
    return float(np.max(np.abs(a - n) / (np.maximum(np.abs(a), np.abs(n)) + 1e-12)))


def test_toy_head_projection_gradients_match_fd():
    """Oracle dQ, dK, dV pushed through the projections agree with central
    differences to the order the page prints (1e-7 .. 1e-10, bar 1e-4)."""
    pr = _golden("datatweets_toy_head.json")["printed"]
    t = _toy_head()
    X, Wq, Wk, Wv, G = t["X"], t["Wq"], t["Wk"], t["Wv"], t["G"]
    r = oracle.attn_bwd(X @ Wq, X @ Wk, X @ Wv, G, scale=1.0 / np.sqrt(8))
    # the projection gradients from the oracle's in_proj_bwd, tokens of the
    # two batch items flattened into rows
    T = X.shape[0] * X.shape[1]
    p = oracle.in_proj_bwd(X.reshape(T, -1), Wq, Wk, Wv, r["dq"].reshape(T, -1),
                           r["dk"].reshape(T, -1), r["dv"].reshape(T, -1))
    analytic = {"dWq": p["dw_q"], "dWk": p["dw_k"], "dWv": p["dw_v"],
                "dX": p["dx"].reshape(X.shape)}
    eps = pr["fd_eps"]
    params = {"dWq": "Wq", "dWk": "Wk", "dWv": "Wv", "dX": "X"}
    for gname, pname in params.items():
        p = t[pname]
        num = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            orig = p[idx]
            p[idx] = orig + eps
            lp = _toy_loss(t["X"], t["Wq"], t["Wk"], t["Wv"], G)
            p[idx] = orig - eps
            lm = _toy_loss(t["X"], t["Wq"], t["Wk"], t["Wv"], G)
            p[idx] = orig
            num[idx] = (lp - lm) / (2 * eps)
        err = _max_rel_err(analytic[gname], num)
        assert err < 1e-5, (gname, err)
        # same order of magnitude as the page's printed figure (or better)
        assert err < 100 * max(pr["fd_max_rel_err"][gname], 1e-9), (gname, err)


# ---------------------------------------------------------------- closed forms

def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_zero_qk_noncausal_closed_form():
    """Q = K = 0: P = 1/m, O_i = mean_j V_j, dV_j = (1/m) sum_i dO_i,
    dS_ij = (1/m) dO_i . (V_j - mean V), dQ = dK = 0."""
    n, m, d, dv = 5, 7, 4, 3
    V = _rand((m, dv), 1)
    dO = _rand((n, dv), 2)
    r = oracle.attn_bwd(np.zeros((n, d)), np.zeros((m, d)), V, dO, want_ds=True)
    np.testing.assert_allclose(r["o"], np.tile(V.mean(0), (n, 1)), atol=1e-14)
    np.testing.assert_allclose(r["dv"], np.tile(dO.sum(0) / m, (m, 1)), atol=1e-14)
    np.testing.assert_allclose(r["ds"], (dO @ (V - V.mean(0)).T) / m, atol=1e-14)
    np.testing.assert_allclose(r["lse"], np.full(n, np.log(m)), atol=1e-14)
    assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0)


def test_zero_qk_causal_closed_form():
    """Causal with Q = K = 0: P_ij = 1/(i+1) for j <= i (eulerpad P8), O_i is
    the prefix mean and dV_j = sum_{i >= j} dO_i / (i+1)."""
    n, d, dv = 6, 4, 3
    V = _rand((n, dv), 3)
    dO = _rand((n, dv), 4)
    r = oracle.attn_bwd(np.zeros((n, d)), np.zeros((n, d)), V, dO, causal=True)
    prefix_mean = np.cumsum(V, 0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(r["o"], prefix_mean, atol=1e-14)
    w = dO / np.arange(1, n + 1)[:, None]
    expect_dv = np.cumsum(w[::-1], 0)[::-1]
    np.testing.assert_allclose(r["dv"], expect_dv, atol=1e-14)
    np.testing.assert_allclose(r["lse"], np.log(np.arange(1, n + 1)), atol=1e-14)


def test_single_key_closed_form():
    """m = 1: P = 1, so O_i = V_0, dV_0 = sum_i dO_i, dS = 0, dQ = dK = 0,
    LSE_i = s q_i . k_0."""
    n, d, dv = 4, 5, 3
    Q, K, V, dO = _rand((n, d), 5), _rand((1, d), 6), _rand((1, dv), 7), _rand((n, dv), 8)
    s = 0.37
    r = oracle.attn_bwd(Q, K, V, dO, scale=s)
    np.testing.assert_allclose(r["o"], np.tile(V[0], (n, 1)), atol=1e-14)
    np.testing.assert_allclose(r["dv"][0], dO.sum(0), atol=1e-14)
    np.testing.assert_allclose(r["lse"], s * (Q @ K[0]), atol=1e-14)
    np.testing.assert_allclose(r["dq"], 0, atol=1e-15)
    np.testing.assert_allclose(r["dk"], 0, atol=1e-15)


def test_identical_values_give_zero_score_gradient():
    """All rows of V equal: dP_ij = dO_i . V_0 for every j, so dP - D = 0,
    dS = 0 and dQ = dK = 0 while O_i = V_0."""
    n, m, d, dv = 5, 6, 4, 3
    Q, K, dO = _rand((n, d), 9), _rand((m, d), 10), _rand((n, dv), 11)
    V = np.tile(_rand((1, dv), 12), (m, 1))
    r = oracle.attn_bwd(Q, K, V, dO, want_ds=True)
    np.testing.assert_allclose(r["ds"], 0, atol=1e-14)
    np.testing.assert_allclose(r["dq"], 0, atol=1e-14)
    np.testing.assert_allclose(r["dk"], 0, atol=1e-14)
    np.testing.assert_allclose(r["o"], np.tile(V[0], (n, 1)), atol=1e-14)


def test_causal_first_row_one_hot():
    """Causal row 0 sees only key 0: P_0 is one-hot, its Jacobian
    diag(u) - u u^T is zero (eulerpad P9), so dQ_0 = 0 exactly."""
    n, d = 6, 4
    Q, K, V, dO = (_rand((n, d), s) for s in (13, 14, 15, 16))
    r = oracle.attn_bwd(Q, K, V, dO, causal=True)
    assert np.all(r["dq"][0] == 0.0)
    np.testing.assert_allclose(r["o"][0], V[0], atol=1e-15)


# ---------------------------------------------------------------- library routines

def _torch_autograd(Q, K, V, dO, scale, causal):
    """float64 autograd through torch's softmax: a different road to the same
    gradient (library routines, no hand-written backward)."""
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    s = (q @ k.transpose(-1, -2)) * scale
    if causal:
        n, m = s.shape[-2:]
        mask = torch.ones(n, m, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ v
    o.backward(torch.tensor(dO, dtype=torch.float64))
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("n,m,d,dv,causal,mult", [
    (8, 8, 16, 16, True, 1.0), (9, 13, 8, 4, False, 1.0), (16, 16, 8, 8, True, 3.0),
    (12, 40, 16, 8, False, 3.0), (33, 33, 8, 12, True, 1.0),
])
def test_matches_torch_autograd(n, m, d, dv, causal, mult):
    B, H = 2, 3
    Q = _rand((B, H, n, d), 20, mult)
    K = _rand((B, H, m, d), 21, mult)
    V = _rand((B, H, m, dv), 22)
    dO = _rand((B, H, n, dv), 23)
    s = 1.0 / np.sqrt(d)
    o, dq, dk, dvv = _torch_autograd(Q, K, V, dO, s, causal)
    r = oracle.attn_bwd(Q, K, V, dO, scale=s, causal=causal)
    for name, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dvv)):
        err = np.max(np.abs(r[name] - ref)) / max(np.max(np.abs(ref)), 1e-300)
        assert err < 1e-12, (name, err)
    # LSE against scipy's logsumexp of the masked scores
    from scipy.special import logsumexp
    S = np.einsum("bhid,bhjd->bhij", Q, K) * s
    if causal:
        S = np.where(np.triu(np.ones((n, m), bool), 1), -np.inf, S)
    np.testing.assert_allclose(r["lse"], logsumexp(S, axis=-1), rtol=1e-13, atol=1e-13)


def test_explicit_jacobian_row():
    """datatweets Exercise 2 / eulerpad P4: applying J = diag(p) - p p^T,
    built explicitly, to the row of dP gives the oracle's dS row."""
    from scipy.special import softmax
    n, m, d, dv = 4, 9, 6, 5
    Q, K, V, dO = _rand((n, d), 30), _rand((m, d), 31), _rand((m, dv), 32), _rand((n, dv), 33)
    s = 1.0 / np.sqrt(d)
    r = oracle.attn_bwd(Q, K, V, dO, scale=s, want_ds=True)
    for i in range(n):
        p = softmax(s * (K @ Q[i]))
        J = np.diag(p) - np.outer(p, p)
        g = V @ dO[i]          # row i of dP, one dot product per key
        np.testing.assert_allclose(J @ g, r["ds"][i], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, n, d, dv = 2, 2, 11, 8, 6
    m = n if causal else 17
    Q, K = _rand((B, H, n, d), 40, 2.0), _rand((B, H, m, d), 41, 2.0)
    V, dO = _rand((B, H, m, dv), 42), _rand((B, H, n, dv), 43)
    r = oracle.attn_bwd(Q, K, V, dO, causal=causal, want_ds=True)
    # I1 each row of dS sums to zero (rows of P sum to 1)
    assert np.max(np.abs(r["ds"].sum(-1))) < 1e-13
    # I2 sum_j dK_j = 0
    assert np.max(np.abs(r["dk"].sum(-2))) < 1e-12
    # I3 sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(r["dv"].sum(-2), dO.sum(-2), atol=1e-12)
    # I4 <Q, dQ> = <K, dK>: S is bilinear in Q and K
    np.testing.assert_allclose((Q * r["dq"]).sum((-1, -2)), (K * r["dk"]).sum((-1, -2)), atol=1e-12)
    # I5 <V, dV> = <O, dO> = sum_i D_i: O is linear in V
    np.testing.assert_allclose((V * r["dv"]).sum((-1, -2)), (r["o"] * dO).sum((-1, -2)), atol=1e-12)
    np.testing.assert_allclose(r["D"].sum(-1), (r["o"] * dO).sum((-1, -2)), atol=1e-12)
    # I6 rowsum(dP o P) = rowsum(dO o O)
    np.testing.assert_allclose(r["D"], r["D_alt"], rtol=1e-12, atol=1e-13)


def test_causal_future_keys_do_not_reach_outputs():
    """I7: perturbing K_j or V_j for j > i leaves O_i unchanged (the mask is
    applied before the softmax, eulerpad mistake 5)."""
    n, d, dv = 7, 4, 3
    Q, K, V = _rand((n, d), 50), _rand((n, d), 51), _rand((n, dv), 52)
    o0, _ = oracle.attn_fwd(Q, K, V, causal=True)
    K2, V2 = K.copy(), V.copy()
    K2[4:] += 10.0
    V2[4:] -= 7.0
    o1, _ = oracle.attn_fwd(Q, K2, V2, causal=True)
    assert np.array_equal(o0[:4], o1[:4])
    assert not np.allclose(o0[4:], o1[4:])


def test_key_permutation_equivariance():
    """I12: permuting keys and values together permutes dK and dV rows and
    leaves O, LSE and dQ unchanged (non-causal)."""
    n, m, d, dv = 5, 9, 4, 3
    Q, K, V, dO = _rand((n, d), 60), _rand((m, d), 61), _rand((m, dv), 62), _rand((n, dv), 63)
    perm = np.random.default_rng(64).permutation(m)
    a = oracle.attn_bwd(Q, K, V, dO)
    b = oracle.attn_bwd(Q, K[perm], V[perm], dO)
    np.testing.assert_allclose(b["o"], a["o"], atol=1e-14)
    np.testing.assert_allclose(b["dq"], a["dq"], atol=1e-14)
    np.testing.assert_allclose(b["dk"], a["dk"][perm], atol=1e-14)
    np.testing.assert_allclose(b["dv"], a["dv"][perm], atol=1e-14)


def test_large_logits_stay_finite():
    """Scores of size about 100 (mlgrind 'Edge cases'): the row max is
    subtracted, so nothing overflows and P rows still sum to one."""
    n, m, d, dv = 6, 10, 16, 4
    Q, K = _rand((n, d), 70, 30.0), _rand((m, d), 71, 30.0)
    V, dO = _rand((m, dv), 72), _rand((n, dv), 73)
    r = oracle.attn_bwd(Q, K, V, dO, scale=1.0, want_ds=True)
    for key in ("o", "lse", "dq", "dk", "dv", "ds"):
        assert np.all(np.isfinite(r[key])), key
    assert np.max(np.abs(r["ds"].sum(-1))) < 1e-9 * max(1.0, np.max(np.abs(r["ds"])))


# ---------------------------------------------------------------- sampled routines

@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_cols_match_full(causal):
    n, d, dv = 37, 8, 6
    m = n if causal else 23
    Q, K, V, dO = _rand((n, d), 80), _rand((m, d), 81), _rand((m, dv), 82), _rand((n, dv), 83)
    full = oracle.attn_bwd(Q, K, V, dO, causal=causal)
    rows = [0, 5, n - 1, 17]
    cols = [0, 3, m - 1, 11]
    a = oracle.attn_rows(Q, K, V, dO, rows, causal=causal)
    b = oracle.attn_cols(Q, K, V, dO, cols, causal=causal)
    np.testing.assert_allclose(a["o"], full["o"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a["lse"], full["lse"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a["D"], full["D"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a["dq"], full["dq"][rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dk"], full["dk"][cols], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dv"], full["dv"][cols], rtol=1e-12, atol=1e-14)


def test_invalid_sizes_rejected():
    with pytest.raises(ValueError):
        oracle.attn_fwd(np.zeros((3, 4)), np.zeros((4, 4)), np.zeros((4, 2)), causal=True)
    with pytest.raises(ValueError):
        oracle.attn_bwd(np.zeros((3, 4)), np.zeros((0, 4)), np.zeros((0, 2)), np.zeros((3, 2)))

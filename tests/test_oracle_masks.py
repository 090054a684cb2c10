"""Pins of the oracle's masked, variable-length routine
(``oracle.attn_bwd_masked``).

The pages fix only the causal mask with n == m; per-batch lengths and the
two causal alignments for n != m are readings (key j visible from row i
when j <= i, "top-left", or j <= i + nk - nq, "bottom-right"; rows that see
no key get zero weights).  Each check below reaches the same numbers by a
different road: the already pinned dense routine on sliced tensors, float64
torch autograd through a mask matrix built from the stated rule, scipy's
logsumexp, closed forms for Q = K = 0, central differences and gradient
invariants.  A last test shows that the autograd check tells the two
alignments apart.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _visible(nb, mb, mask):
    """[nb, mb] boolean matrix of the stated rule."""
    i = np.arange(nb)[:, None]
    j = np.arange(mb)[None, :]
    if mask == "none":
        return np.ones((nb, mb), bool)
    off = 0 if mask == "causal" else mb - nb
    return j <= i + off


def _autograd(Q, K, V, dO, scale, vis):
    """float64 torch autograd of softmax(S with -inf where not visible) V.
    Rows with no visible key are left out (their softmax is 0/0)."""
    rows = vis.any(1)
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    s = (q @ k.T) * scale
    s = s.masked_fill(torch.from_numpy(~vis), float("-inf"))
    r = torch.from_numpy(rows)
    o = torch.softmax(s[r], dim=-1) @ v
    o.backward(torch.tensor(dO[rows], dtype=torch.float64))
    lse = torch.logsumexp(s[r], dim=-1)
    return rows, o.detach().numpy(), lse.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def test_full_lengths_reduce_to_dense_routine():
    """No lengths, mask 'causal' with n == m and mask 'none' with n != m are
    the pages' problems: identical to the dense routine."""
    B, H, n, d, dv = 2, 2, 13, 8, 6
    for mask, m in (("causal", n), ("none", 21), ("causal_bottom_right", n)):
        Q, K = _rand((B, H, n, d), 1), _rand((B, H, m, d), 2)
        V, dO = _rand((B, H, m, dv), 3), _rand((B, H, n, dv), 4)
        a = oracle.attn_bwd_masked(Q, K, V, dO, mask=mask)
        b = oracle.attn_bwd(Q, K, V, dO, causal=(mask != "none"))
        for key in ("o", "lse", "dq", "dk", "dv", "D"):
            np.testing.assert_allclose(a[key], b[key], rtol=1e-13, atol=1e-14, err_msg=(mask, key))


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_lengths_equal_dense_routine_on_slices(mask):
    """Batch b with lengths (nq[b], nk[b]) is the dense problem on the first
    nq[b] query rows and nk[b] key rows; padding rows are zero (LSE -inf)."""
    B, H, n, m, d, dv = 4, 2, 17, 17, 8, 5
    Q, K = _rand((B, H, n, d), 10), _rand((B, H, m, d), 11)
    V, dO = _rand((B, H, m, dv), 12), _rand((B, H, n, dv), 13)
    lq = [17, 9, 1, 12]
    lk = [17, 9, 1, 12] if mask == "causal" else [3, 17, 8, 1]
    r = oracle.attn_bwd_masked(Q, K, V, dO, mask=mask, seqlens_q=lq, seqlens_k=lk)
    for b in range(B):
        nb, mb = lq[b], lk[b]
        ref = oracle.attn_bwd(Q[b:b + 1, :, :nb], K[b:b + 1, :, :mb], V[b:b + 1, :, :mb],
                              dO[b:b + 1, :, :nb], causal=(mask == "causal"))
        for key, rows in (("o", nb), ("lse", nb), ("dq", nb), ("D", nb), ("dk", mb), ("dv", mb)):
            np.testing.assert_allclose(r[key][b:b + 1, :, :rows], ref[key], rtol=1e-13,
                                       atol=1e-14, err_msg=(b, key))
        assert np.all(r["o"][b, :, nb:] == 0) and np.all(r["dq"][b, :, nb:] == 0)
        assert np.all(r["lse"][b, :, nb:] == -np.inf) and np.all(r["D"][b, :, nb:] == 0)
        assert np.all(r["dk"][b, :, mb:] == 0) and np.all(r["dv"][b, :, mb:] == 0)


@pytest.mark.parametrize("mask", ["causal", "causal_bottom_right"])
@pytest.mark.parametrize("nb,mb", [(7, 12), (12, 7), (9, 9), (5, 1), (1, 6)])
def test_causal_alignments_match_autograd(mask, nb, mb):
    d, dv, s = 8, 5, 0.4
    Q, K = _rand((nb, d), 20 + nb, 2.0), _rand((mb, d), 21 + mb, 2.0)
    V, dO = _rand((mb, dv), 22), _rand((nb, dv), 23)
    vis = _visible(nb, mb, mask)
    rows, o, lse, dq, dk, dvv = _autograd(Q, K, V, dO, s, vis)
    r = oracle.attn_bwd_masked(Q[None, None], K[None, None], V[None, None], dO[None, None],
                               scale=s, mask=mask)
    r = {key: val[0, 0] for key, val in r.items()}
    np.testing.assert_allclose(r["o"][rows], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["lse"][rows], lse, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dq"], dq, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["dk"], dk, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["dv"], dvv, rtol=1e-11, atol=1e-13)
    # rows that see no key: zero weights
    assert np.all(r["o"][~rows] == 0) and np.all(r["dq"][~rows] == 0)
    assert np.all(r["lse"][~rows] == -np.inf)
    # LSE against scipy's logsumexp of the masked scores
    from scipy.special import logsumexp
    S = np.where(vis, s * Q @ K.T, -np.inf)
    np.testing.assert_allclose(r["lse"][rows], logsumexp(S[rows], axis=-1), rtol=1e-13)


def test_alignments_are_told_apart():
    """Negative control: with nq != nk, the top-left routine does not pass
    the bottom-right autograd check and vice versa."""
    nb, mb, d, dv = 6, 10, 8, 4
    Q, K, V, dO = _rand((nb, d), 30), _rand((mb, d), 31), _rand((mb, dv), 32), _rand((nb, dv), 33)
    for routine, other in (("causal", "causal_bottom_right"), ("causal_bottom_right", "causal")):
        _, o, _, _, _, _ = _autograd(Q, K, V, dO, 0.3, _visible(nb, mb, other))
        r = oracle.attn_bwd_masked(Q[None, None], K[None, None], V[None, None], dO[None, None],
                                   scale=0.3, mask=routine)
        assert np.max(np.abs(r["o"][0, 0] - o)) > 1e-2


def test_bottom_right_zero_qk_closed_form():
    """Q = K = 0 under the bottom-right mask with nk > nq: row i averages the
    first i + nk - nq + 1 values, and dV_j = sum over rows that see j of
    dO_i / (i + nk - nq + 1); LSE_i = ln(i + nk - nq + 1); dQ = dK = 0."""
    nb, mb, d, dv = 5, 9, 4, 3
    V, dO = _rand((mb, dv), 40), _rand((nb, dv), 41)
    r = oracle.attn_bwd_masked(np.zeros((1, 1, nb, d)), np.zeros((1, 1, mb, d)), V[None, None],
                               dO[None, None], mask="causal_bottom_right")
    cnt = np.arange(nb) + (mb - nb) + 1
    o_ref = np.stack([V[:c].mean(0) for c in cnt])
    dv_ref = np.zeros((mb, dv))
    for i, c in enumerate(cnt):
        dv_ref[:c] += dO[i] / c
    np.testing.assert_allclose(r["o"][0, 0], o_ref, atol=1e-14)
    np.testing.assert_allclose(r["dv"][0, 0], dv_ref, atol=1e-14)
    np.testing.assert_allclose(r["lse"][0, 0], np.log(cnt), atol=1e-14)
    assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0)


def test_bottom_right_finite_differences():
    """Central differences of L = sum(O o dO) (eps = 1e-5, float64), with
    nq > nk so that the first rows see no key."""
    nb, mb, d, dv, eps = 6, 4, 3, 2, 1e-5
    Q, K, V, dO = _rand((nb, d), 50), _rand((mb, d), 51), _rand((mb, dv), 52), _rand((nb, dv), 53)

    def loss():
        r = oracle.attn_bwd_masked(Q[None, None], K[None, None], V[None, None], dO[None, None],
                                   mask="causal_bottom_right")
        return float(np.sum(r["o"] * dO[None, None]))

    r = oracle.attn_bwd_masked(Q[None, None], K[None, None], V[None, None], dO[None, None],
                               mask="causal_bottom_right")
    for name, T in (("dq", Q), ("dk", K), ("dv", V)):
        g = np.zeros_like(T)
        for idx in np.ndindex(T.shape):
            orig = T[idx]
            T[idx] = orig + eps
            lp = loss()
            T[idx] = orig - eps
            lm = loss()
            T[idx] = orig
            g[idx] = (lp - lm) / (2 * eps)
        a = r[name][0, 0]
        np.testing.assert_allclose(a, g, rtol=1e-6, atol=1e-8, err_msg=name)


def test_masked_invariants_per_batch():
    """With lengths and the bottom-right mask: sum_j dK_j = 0 and
    sum_j dV_j = sum of dO over rows that see a key, <Q,dQ> = <K,dK>,
    <V,dV> = <O,dO>."""
    B, H, n, m, d, dv = 3, 2, 11, 14, 6, 5
    Q, K = _rand((B, H, n, d), 60, 2.0), _rand((B, H, m, d), 61, 2.0)
    V, dO = _rand((B, H, m, dv), 62), _rand((B, H, n, dv), 63)
    lq, lk = [11, 8, 6], [14, 3, 6]
    r = oracle.attn_bwd_masked(Q, K, V, dO, mask="causal_bottom_right", seqlens_q=lq,
                               seqlens_k=lk)
    for b in range(B):
        seen = np.isfinite(r["lse"][b, 0])          # rows that see a key
        np.testing.assert_allclose(r["dk"][b].sum(-2), 0, atol=1e-12)
        np.testing.assert_allclose(r["dv"][b].sum(-2), dO[b][:, seen].sum(-2), atol=1e-12)
        np.testing.assert_allclose((Q[b] * r["dq"][b]).sum((-1, -2)),
                                   (K[b] * r["dk"][b]).sum((-1, -2)), atol=1e-12)
        np.testing.assert_allclose((V[b] * r["dv"][b]).sum((-1, -2)),
                                   (r["o"][b] * dO[b]).sum((-1, -2)), atol=1e-12)


@pytest.mark.parametrize("off", [-3, 0, 4])
def test_sampled_routines_follow_the_offset(off):
    """attn_rows / attn_cols with a causal offset agree with the full masked
    routine (bottom-right mask, nk - nq = off)."""
    n, d, dv = 15, 6, 4
    m = n + off
    Q, K, V, dO = _rand((n, d), 70), _rand((m, d), 71), _rand((m, dv), 72), _rand((n, dv), 73)
    full = oracle.attn_bwd_masked(Q[None, None], K[None, None], V[None, None], dO[None, None],
                                  mask="causal_bottom_right")
    full = {key: val[0, 0] for key, val in full.items()}
    rows = [0, 1, 2, 3, 7, n - 1]
    cols = [0, 2, m - 1]
    a = oracle.attn_rows(Q, K, V, dO, rows, causal=True, causal_offset=off)
    b = oracle.attn_cols(Q, K, V, dO, cols, causal=True, causal_offset=off)
    np.testing.assert_allclose(a["o"], full["o"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(np.isinf(a["lse"]), np.isinf(full["lse"][rows]))
    fin = np.isfinite(a["lse"])
    np.testing.assert_allclose(a["lse"][fin], full["lse"][rows][fin], rtol=1e-13)
    np.testing.assert_allclose(a["dq"], full["dq"][rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dk"], full["dk"][cols], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dv"], full["dv"][cols], rtol=1e-12, atol=1e-14)


def test_masked_invalid_arguments():
    z = np.zeros((1, 1, 3, 4))
    with pytest.raises(ValueError):
        oracle.attn_bwd_masked(z, z, z, z, seqlens_q=[1, 2])
    with pytest.raises(KeyError):
        oracle.attn_bwd_masked(z, z, z, z, mask="sliding")

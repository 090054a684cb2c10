"""Pins of the oracle's projection gradients (eulerpad "Attention backward"
Problems 7 and 10; datatweets "Step 4"): a whole multi-head self-attention
layer Y = concat_h(attention(X W_Q,h, X W_K,h, X W_V,h)) W_O is
differentiated by the oracle's chain (out_proj_bwd, the per-head attention
backward, in_proj_bwd) and checked against central differences of
L = sum(Y o G) in float64, for every entry of X, W_Q, W_K, W_V and W_O.
The toy head of the datatweets lesson pins in_proj_bwd to the page's
printed figures (tests/test_oracle_pins.py).
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _layer(X, Wq, Wk, Wv, Wo, B, n, H, d, dv, causal):
    """Forward of the layer: per-head attention on the column blocks."""
    T = B * n
    Q, K, V = X @ Wq, X @ Wk, X @ Wv                     # [T, H d], [T, H d], [T, H dv]
    heads = lambda M, w: M.reshape(B, n, H, w).transpose(0, 2, 1, 3)   # [B, H, n, w]
    o, _ = oracle.attn_fwd(heads(Q, d), heads(K, d), heads(V, dv), causal=causal)
    o_cat = o.transpose(0, 2, 1, 3).reshape(T, H * dv)
    return o_cat @ Wo, o_cat


def _grads(X, Wq, Wk, Wv, Wo, G, B, n, H, d, dv, causal):
    T = B * n
    Y, o_cat = _layer(X, Wq, Wk, Wv, Wo, B, n, H, d, dv, causal)
    a = oracle.out_proj_bwd(o_cat, G, Wo)
    heads = lambda M, w: M.reshape(B, n, H, w).transpose(0, 2, 1, 3)
    cat = lambda M: M.transpose(0, 2, 1, 3).reshape(T, -1)
    r = oracle.attn_bwd(heads(X @ Wq, d), heads(X @ Wk, d), heads(X @ Wv, dv),
                        heads(a["do_cat"], dv), causal=causal)
    b = oracle.in_proj_bwd(X, Wq, Wk, Wv, cat(r["dq"]), cat(r["dk"]), cat(r["dv"]))
    return {"X": b["dx"], "Wq": b["dw_q"], "Wk": b["dw_k"], "Wv": b["dw_v"], "Wo": a["dw_o"]}


@pytest.mark.parametrize("causal", [False, True])
def test_layer_gradients_match_finite_differences(causal):
    B, n, H, d, dv, dm = 2, 5, 2, 3, 4, 6
    T = B * n
    P = {"X": _rand((T, dm), 1), "Wq": _rand((dm, H * d), 2, 0.5),
         "Wk": _rand((dm, H * d), 3, 0.5), "Wv": _rand((dm, H * dv), 4, 0.5),
         "Wo": _rand((H * dv, dm), 5, 0.5)}
    G = _rand((T, dm), 6)
    shape = (B, n, H, d, dv, causal)
    analytic = _grads(P["X"], P["Wq"], P["Wk"], P["Wv"], P["Wo"], G, *shape)

    def loss():
        Y, _ = _layer(P["X"], P["Wq"], P["Wk"], P["Wv"], P["Wo"], *shape)
        return float(np.sum(Y * G))

    eps = 1e-5
    for name, p in P.items():
        num = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            orig = p[idx]
            p[idx] = orig + eps
            lp = loss()
            p[idx] = orig - eps
            lm = loss()
            p[idx] = orig
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(analytic[name] - num)) / np.max(np.abs(num))
        assert err < 1e-7, (name, err)


def test_out_proj_slices_are_head_gradients():
    """Problem 10: column block h of G W_O^T is the gradient of head h's
    output, i.e. what G W_O^T restricted to W_O's row block h gives."""
    T, H, dv, dm = 7, 3, 4, 5
    o_cat, G, Wo = _rand((T, H * dv), 10), _rand((T, dm), 11), _rand((H * dv, dm), 12)
    a = oracle.out_proj_bwd(o_cat, G, Wo)
    for h in range(H):
        blk = slice(h * dv, (h + 1) * dv)
        np.testing.assert_allclose(a["do_cat"][:, blk], G @ Wo[blk].T, rtol=1e-14, atol=1e-14)
        # and dW_O's row block h only sees head h's output
        np.testing.assert_allclose(a["dw_o"][blk], o_cat[:, blk].T @ G, rtol=1e-14, atol=1e-14)

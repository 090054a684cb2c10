"""Central finite differences pin the oracle's backward to its forward, and
the known-wrong formulas from the pages fail the same check.

The gradient check is the datatweets lesson's ('Proving It: A Numerical
Gradient Check'): eps = 1e-5 in float64, metric max |a - n| / max(|a|, |n|).
The loss is L = sum(O o dO), whose gradient with respect to O is dO exactly
(mlgrind 'Edge cases'; datatweets 'A Scalar Loss So dout Is Known').
"""
import numpy as np
import pytest

import oracle

EPS = 1e-5


def _loss(Q, K, V, dO, scale, causal):
    o, _ = oracle.attn_fwd(Q, K, V, scale=scale, causal=causal)
    return float(np.sum(o * dO))


def _fd_grads(Q, K, V, dO, scale, causal):
    out = {}
    for name, T in (("dq", Q), ("dk", K), ("dv", V)):
        g = np.zeros_like(T)
        for idx in np.ndindex(T.shape):
            orig = T[idx]
            T[idx] = orig + EPS
            lp = _loss(Q, K, V, dO, scale, causal)
            T[idx] = orig - EPS
            lm = _loss(Q, K, V, dO, scale, causal)
            T[idx] = orig
            g[idx] = (lp - lm) / (2 * EPS)
        out[name] = g
    return out


def _err(a, n):
    """Relative error where the gradient is not tiny, absolute below 1e-9
    (for example the causal first row of dQ, which is exactly zero)."""
    big = np.maximum(np.abs(a), np.abs(n))
    rel = np.abs(a - n) / (big + 1e-12)
    rel = np.where(big < 1e-9, np.abs(a - n), rel)
    return float(np.max(rel))


CASES = [
    # (n, m, d, dv, causal, logit multiplier)
    (2, 3, 4, 2, False, 1.0),
    (3, 3, 4, 4, True, 1.0),
    (5, 7, 4, 3, False, 1.0),
    (8, 8, 8, 8, True, 1.0),
    (4, 6, 8, 2, False, 30.0),
]


def _inputs(n, m, d, dv, mult, seed=0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((n, d)) * mult
    K = rng.standard_normal((m, d)) * mult
    V = rng.standard_normal((m, dv))
    dO = rng.standard_normal((n, dv))
    return Q, K, V, dO


@pytest.mark.parametrize("n,m,d,dv,causal,mult", CASES)
def test_backward_matches_finite_differences(n, m, d, dv, causal, mult):
    Q, K, V, dO = _inputs(n, m, d, dv, mult)
    # with logits x30 the scores reach hundreds; use s = 1/sqrt(d) throughout
    s = 1.0 / np.sqrt(d)
    r = oracle.attn_bwd(Q, K, V, dO, scale=s, causal=causal)
    fd = _fd_grads(Q, K, V, dO, s, causal)
    for name in ("dq", "dk", "dv"):
        e = _err(r[name], fd[name])
        assert e < 1e-5, (name, e)


# Each known-wrong formula must fail the check clearly (the page calls
# ~1e-2 "a real bug").  Cases chosen so that each mistake is visible.
MUTANT_CASES = {
    "ds_no_correction": (5, 7, 4, 3, False),
    "ds_diag_only": (5, 7, 4, 3, False),
    "dv_no_transpose": (6, 6, 4, 3, False),
    "flat_jacobian": (5, 7, 4, 3, False),
    "drop_scale": (5, 7, 16, 3, False),
    "mask_after_softmax": (6, 6, 4, 3, True),
}


@pytest.mark.parametrize("name", sorted(MUTANT_CASES))
def test_known_wrong_variants_fail(name):
    n, m, d, dv, causal = MUTANT_CASES[name]
    Q, K, V, dO = _inputs(n, m, d, dv, 1.0, seed=1)
    s = 1.0 / np.sqrt(d)
    fd = _fd_grads(Q, K, V, dO, s, causal)
    good = oracle.attn_bwd(Q, K, V, dO, scale=s, causal=causal)
    bad = oracle.attn_bwd(Q, K, V, dO, scale=s, causal=causal,
                          variant=oracle.WRONG_VARIANTS[name])
    worst_good = max(_err(good[t], fd[t]) for t in ("dq", "dk", "dv"))
    worst_bad = max(_err(bad[t], fd[t]) for t in ("dq", "dk", "dv"))
    assert worst_good < 1e-5
    assert worst_bad > 1e-2, (name, worst_bad)

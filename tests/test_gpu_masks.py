"""GPU parity for masks beyond causal n == m: per-batch sequence lengths and
the two causal alignments (top-left j <= i, bottom-right j <= i + m_b - n_b),
through attn_fwd_ex / attn_bwd_ex, against the oracle's masked routine.

Padded rows of the inputs are filled with NaN: the kernels must never read
them, and the outputs there must be exact zeros (LSE -inf).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attn_bwd_amd as attn

from gpu_util import TOL, rel_err, say, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
LSE_TOL = {"bf16": 1e-3, "fp16": 1e-3, "fp32": 1e-5}


def _inputs(B, H, n, m, d, dv, dtype, seed, lq, lk, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, n, d), generator=g) * mult
    k = torch.randn((B, H, m, d), generator=g) * mult
    v = torch.randn((B, H, m, dv), generator=g)
    do = torch.randn((B, H, n, dv), generator=g)
    q, k, v, do = (t.to(DT[dtype]) for t in (q, k, v, do))
    for b in range(B):
        nb = n if lq is None else lq[b]
        mb = m if lk is None else lk[b]
        q[b, :, nb:] = float("nan")
        do[b, :, nb:] = float("nan")
        k[b, :, mb:] = float("nan")
        v[b, :, mb:] = float("nan")
    return q, k, v, do


def _run(case, layout="bhsd", scale=None):
    (name, B, H, n, m, d, dv, dtype, mask, lq, lk, seed) = case
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"case {name}: B={B} H={H} n={n} m={m} d={d} dv={dv} {dtype} mask={mask} lq={lq} "
        f"lk={lk} layout={layout} scale={scale}")
    q, k, v, do = _inputs(B, H, n, m, d, dv, dtype, seed, lq, lk)
    dev = "cuda:0"
    # [B, seq, H, dim] copies for the bshd layout; results are viewed back
    # as [B, H, seq, dim] for the comparison
    to_dev = (lambda t: t.transpose(1, 2).contiguous().to(dev)) if layout == "bshd" else \
        (lambda t: t.to(dev))
    back = (lambda t: t.transpose(1, 2)) if layout == "bshd" else (lambda t: t)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    sq = torch.tensor(lq, dtype=torch.int32, device=dev) if lq is not None else None
    sk = torch.tensor(lk, dtype=torch.int32, device=dev) if lk is not None else None
    o, lse = attn.fwd(qd, kd, vd, scale=scale, mask=mask, seqlens_q=sq, seqlens_k=sk,
                      layout=layout)
    dq, dk, dvv = attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, mask=mask, seqlens_q=sq,
                           seqlens_k=sk, layout=layout)
    torch.cuda.synchronize()
    o, dq, dk, dvv = back(o), back(dq), back(dk), back(dvv)
    ref = oracle.attn_bwd_masked(torch.nan_to_num(q), torch.nan_to_num(k), torch.nan_to_num(v),
                                 torch.nan_to_num(do), scale=scale, mask=mask,
                                 seqlens_q=lq, seqlens_k=lk)
    got = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dvv}
    errs = {}
    for key in ("o", "dq", "dk", "dv"):
        g64 = to64(got[key])
        assert np.all(np.isfinite(g64)), (name, key, "non-finite output")
        errs[key] = rel_err(g64, ref[key])
    g_lse = to64(lse)
    assert np.array_equal(np.isneginf(g_lse), np.isneginf(ref["lse"])), (name, "lse -inf pattern")
    fin = np.isfinite(ref["lse"])
    errs["lse_abs"] = float(np.max(np.abs(g_lse[fin] - ref["lse"][fin]))) if fin.any() else 0.0
    say("  errors " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in errs.items()))
    for key in ("o", "dq", "dk", "dv"):
        assert errs[key] <= TOL[dtype], (name, key, errs[key])
    assert errs["lse_abs"] <= LSE_TOL[dtype], (name, "lse", errs["lse_abs"])
    # exact zeros where the problem has no rows
    for b in range(B):
        nb = n if lq is None else lq[b]
        mb = m if lk is None else lk[b]
        assert torch.count_nonzero(o[b, :, nb:]) == 0 and torch.count_nonzero(dq[b, :, nb:]) == 0
        assert torch.count_nonzero(dk[b, :, mb:]) == 0 and torch.count_nonzero(dvv[b, :, mb:]) == 0


CASES = [
    # name, B, H, n, m, d, dv, dtype, mask, seqlens_q, seqlens_k, seed
    ("varlen_none_d128", 4, 2, 300, 300, 128, 128, "bf16", "none",
     [300, 17, 0, 256], [300, 1, 129, 255], 101),
    ("varlen_causal_d128", 4, 2, 600, 600, 128, 128, "bf16", "causal",
     [600, 64, 1, 257], [600, 64, 1, 257], 102),
    ("topleft_n200_m333", 1, 2, 200, 333, 128, 64, "bf16", "causal", None, None, 103),
    ("topleft_n333_m200", 1, 2, 333, 200, 64, 64, "bf16", "causal", None, None, 104),
    ("bottomright_n200_m700", 1, 2, 200, 700, 128, 128, "bf16", "causal_bottom_right",
     None, None, 105),
    ("bottomright_n700_m200", 1, 2, 700, 200, 128, 128, "bf16", "causal_bottom_right",
     None, None, 106),
    ("bottomright_varlen", 3, 2, 500, 600, 128, 128, "bf16", "causal_bottom_right",
     [130, 500, 64], [600, 90, 64], 107),
    ("bottomright_varlen_d64", 3, 1, 300, 300, 64, 64, "bf16", "causal_bottom_right",
     [300, 45, 250], [33, 300, 251], 108),
    ("bottomright_varlen_dv64", 2, 2, 257, 513, 128, 64, "bf16", "causal_bottom_right",
     [257, 100], [513, 160], 109),
    ("varlen_causal_fp16", 3, 2, 400, 400, 128, 128, "fp16", "causal_bottom_right",
     [400, 7, 300], [390, 7, 333], 110),
    ("varlen_none_fp32", 3, 1, 70, 90, 48, 40, "fp32", "none", [70, 0, 33], [90, 5, 0], 111),
    ("bottomright_fp32", 2, 1, 65, 40, 64, 32, "fp32", "causal_bottom_right",
     [65, 20], [40, 40], 112),
    ("topleft_fp32", 1, 2, 30, 77, 100, 20, "fp32", "causal", None, None, 113),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_masked_parity(case):
    _run(case)


SCALE_CASES = [
    (("zero_scale_br_varlen", 3, 2, 300, 400, 128, 128, "bf16", "causal_bottom_right",
      [300, 120, 77], [400, 64, 200], 150), 0.0),
    (("zero_scale_topleft_fp16", 2, 1, 257, 257, 64, 64, "fp16", "causal", [257, 100],
      [257, 130], 151), 0.0),
    (("negative_scale_br_varlen", 2, 2, 333, 257, 128, 64, "bf16", "causal_bottom_right",
      [333, 90], [257, 200], 152), -0.07),
]


@pytest.mark.parametrize("case,scale", SCALE_CASES,
                         ids=lambda c: c[0] if isinstance(c, tuple) else str(c))
def test_masked_zero_and_negative_scale(case, scale):
    """Masks and lengths with a zero scale (every visible weight equal: the
    forward must keep masked and padded logits at -inf, not -inf * 0) and a
    negative one (the forward negates Q)."""
    _run(case, scale=scale)


BSHD_CASES = [
    ("bshd_causal_d128", 2, 3, 300, 300, 128, 128, "bf16", "causal", None, None, 140),
    ("bshd_none_d64_dv128", 1, 4, 130, 333, 64, 128, "bf16", "none", None, None, 141),
    ("bshd_varlen_br_d96", 3, 2, 400, 500, 96, 96, "bf16", "causal_bottom_right",
     [400, 33, 250], [500, 90, 250], 142),
    ("bshd_fp16_d128_dv64", 2, 2, 257, 257, 128, 64, "fp16", "causal", [257, 200], [257, 200],
     143),
    ("bshd_fp32", 2, 3, 50, 70, 40, 24, "fp32", "causal_bottom_right", [50, 20], [70, 31], 144),
]


@pytest.mark.parametrize("case", BSHD_CASES, ids=lambda c: c[0])
def test_bshd_layout_parity(case):
    """[B, seq, H, dim] tensors (what a fused projection produces): same
    results as the oracle on the [B, H, seq, dim] view."""
    _run(case, layout="bshd")


def test_full_lengths_match_plain_entry_points():
    """Lengths equal to n and m, causal: identical bits to attn_fwd/attn_bwd."""
    dev = "cuda:0"
    B, H, n, d = 2, 2, 300, 128
    q, k, v, do = _inputs(B, H, n, n, d, d, "bf16", 120, None, None)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    full = torch.full((B,), n, dtype=torch.int32, device=dev)
    o1, l1 = attn.fwd(q, k, v, causal=True)
    o2, l2 = attn.fwd(q, k, v, mask="causal_bottom_right", seqlens_q=full, seqlens_k=full)
    g1 = attn.bwd(q, k, v, o1, do, l1, causal=True)
    g2 = attn.bwd(q, k, v, o2, do, l2, mask="causal_bottom_right", seqlens_q=full,
                  seqlens_k=full)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_lengths_outside_range_are_clamped():
    """Lengths beyond n or m act as n or m; negative ones as 0."""
    dev = "cuda:0"
    B, H, n, m, d = 2, 1, 100, 130, 64
    q, k, v, do = _inputs(B, H, n, m, d, d, "bf16", 121, None, None)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    big = torch.tensor([1000, -5], dtype=torch.int32, device=dev)
    bigk = torch.tensor([10**6, -1], dtype=torch.int32, device=dev)
    o, lse = attn.fwd(q, k, v, mask="none", seqlens_q=big, seqlens_k=bigk)
    o_ref, lse_ref = attn.fwd(q[:1], k[:1], v[:1])
    torch.cuda.synchronize()
    assert torch.equal(o[:1], o_ref) and torch.equal(lse[:1], lse_ref)
    assert torch.count_nonzero(o[1]) == 0 and bool(torch.all(torch.isneginf(lse[1])))


def test_varlen_bottom_right_4k_sampled():
    """A larger mix of lengths (B=4, H=16, up to 4096 rows, d=128, bf16,
    bottom-right causal): sampled query rows and key rows of three heads
    per batch element against the oracle's sampled routines on the sliced
    problem, whose causal offset is m_b - n_b."""
    dev = "cuda:0"
    B, H, n, m, d = 4, 16, 4096, 4096, 128
    lq, lk = [4096, 3001, 1500, 777], [4096, 3500, 1500, 2000]
    q, k, v, do = _inputs(B, H, n, m, d, d, "bf16", 130, lq, lk)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    sq = torch.tensor(lq, dtype=torch.int32, device=dev)
    sk = torch.tensor(lk, dtype=torch.int32, device=dev)
    scale = 1.0 / np.sqrt(d)
    o, lse = attn.fwd(qd, kd, vd, scale=scale, mask="causal_bottom_right", seqlens_q=sq,
                      seqlens_k=sk)
    dq, dk, dvv = attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, mask="causal_bottom_right",
                           seqlens_q=sq, seqlens_k=sk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    worst = {}
    for b in range(B):
        nb, mb = lq[b], lk[b]
        for h in sorted({0, H - 1, int(rng.integers(H))}):
            Q, K, V, dO = (to64(t[b, h]) for t in (q[:, :, :nb], k[:, :, :mb], v[:, :, :mb],
                                                   do[:, :, :nb]))
            rows = sorted({0, 1, nb // 2, nb - 1, *rng.choice(nb, 8, replace=False).tolist()})
            cols = sorted({0, mb // 2, mb - 1, *rng.choice(mb, 8, replace=False).tolist()})
            r = oracle.attn_rows(Q, K, V, dO, rows, scale=scale, causal=True,
                                 causal_offset=mb - nb)
            c = oracle.attn_cols(Q, K, V, dO, cols, scale=scale, causal=True,
                                 causal_offset=mb - nb)
            errs = {
                "o": rel_err(to64(o[b, h, rows]), r["o"]),
                "dq": rel_err(to64(dq[b, h, rows]), r["dq"]),
                "dk": rel_err(to64(dk[b, h, cols]), c["dk"]),
                "dv": rel_err(to64(dvv[b, h, cols]), c["dv"]),
            }
            fin = np.isfinite(r["lse"])
            assert np.array_equal(np.isneginf(to64(lse[b, h, rows])), ~fin)
            errs["lse_abs"] = float(np.max(np.abs(to64(lse[b, h, rows])[fin] - r["lse"][fin])))
            for key_, val in errs.items():
                worst[key_] = max(worst.get(key_, 0.0), val)
        assert torch.count_nonzero(o[b, :, nb:]) == 0 and torch.count_nonzero(dk[b, :, mb:]) == 0
    say("  worst " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in worst.items()))
    for key_ in ("o", "dq", "dk", "dv"):
        assert worst[key_] <= TOL["bf16"], (key_, worst[key_])
    assert worst["lse_abs"] <= 1e-3

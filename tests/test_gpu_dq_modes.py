"""GPU parity of the ways dQ is accumulated (ATTN_DQ_SEPARATE,
ATTN_DQ_ATOMIC at several splits, ATTN_DQ_STORED_DS and ATTN_DQ_AUTO)
against the float64 oracle, on seeded inputs spanning several 256-key blocks with ragged tails,
every head-width pair, both 16-bit types, masks with per-batch lengths and
the [B, seq, H, dim] layout.

dK and dV do not depend on the dQ mode: the fused and the dS-storing
kernels' dK/dV arithmetic is the plain kernel's, so they must agree bit for
bit across modes.  dQ in the atomic mode is summed in an order the hardware
chooses, and in the stored-dS mode from the dK/dV kernel's dS, so it is held
to the oracle's tolerance and to a tight agreement with the separate pass.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd.workloads import Workload, make_inputs

from gpu_util import LSE_TOL, TOL, oracle_full, rel_err, say, to64

pytestmark = pytest.mark.gpu


def _w(name, B, H, n, m, d, dv, dtype, causal, seed, qk_mult=1.0, scale=None):
    return Workload(name, B, H, n, m, d, dv, dtype, causal, seed, qk_mult, scale)


SHAPES = [
    _w("bf16_causal_700_d128", 1, 2, 700, 700, 128, 128, "bf16", True, 81),
    _w("bf16_causal_1100_d64", 1, 2, 1100, 1100, 64, 64, "bf16", True, 82),
    _w("bf16_cross_300x1000_d128_dv64", 2, 1, 300, 1000, 128, 64, "bf16", False, 83, 3.0),
    _w("bf16_cross_130x530_d64_dv128", 1, 2, 130, 530, 64, 128, "bf16", False, 84),
    _w("bf16_d96_causal_600", 1, 1, 600, 600, 96, 96, "bf16", True, 85),
    _w("bf16_d40_dv72_cross", 1, 1, 100, 777, 40, 72, "bf16", False, 86),
    _w("f16_causal_800_d128", 1, 2, 800, 800, 128, 128, "fp16", True, 87),
    _w("f16_cross_200x600_d128_dv64", 1, 1, 200, 600, 128, 64, "fp16", False, 88, 3.0),
    _w("bf16_single_key_block", 1, 1, 77, 200, 128, 128, "bf16", False, 89),
    _w("bf16_many_heads_causal_520", 4, 16, 520, 520, 128, 128, "bf16", True, 90),
    # degenerate sizes: one query and one key, one ragged 32-row tile on the
    # diagonal, one key for many rows
    _w("bf16_one_query_one_key", 1, 1, 1, 1, 64, 64, "bf16", False, 96),
    _w("bf16_causal_33_d128", 1, 2, 33, 33, 128, 128, "bf16", True, 97),
    _w("bf16_257_queries_one_key", 1, 1, 257, 1, 128, 128, "bf16", False, 98),
]


def _modes(w):
    nkb = (w.m + 255) // 256
    modes = [("separate", None), ("auto", None), ("stored_ds", None), ("atomic", 0),
             ("atomic", 1)]
    if nkb > 2:
        modes.append(("atomic", nkb // 2))
    modes.append(("atomic", nkb))   # every key block in the separate pass
    return modes


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_dq_modes_against_oracle(w):
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    q, k, v, do = (t.to("cuda:0") for t in inputs)
    o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=w.causal)
    ref = oracle_full(w, inputs)
    tol = TOL[w.dtype]
    base = None
    for mode, split in _modes(w):
        dq, dk, dv = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal,
                              dq_mode=mode, dq_split=split)
        torch.cuda.synchronize()
        errs = {n_: rel_err(to64(t), ref[n_]) for n_, t in (("dq", dq), ("dk", dk), ("dv", dv))}
        say(f"  {mode} split={split}: " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in errs.items()))
        for n_, e in errs.items():
            assert e <= tol, (w.name, mode, split, n_, e)
        if base is None:
            base = (dq.clone(), dk.clone(), dv.clone())
        else:
            assert torch.equal(dk, base[1]) and torch.equal(dv, base[2]), (mode, split)
            # the two summation orders of dQ agree to a few 16-bit ulps
            diff = (dq.double() - base[0].double()).abs().max().item()
            assert diff <= tol * 0.25 * base[0].double().abs().max().item(), (mode, split, diff)


def test_atomic_mode_repeats_within_rounding():
    """Two atomic-mode calls on the same inputs give identical dK, dV and
    dQ within a few ulps (float32 atomics commute only up to rounding)."""
    w = SHAPES[0]
    say(f"case repeat {w.describe()}")
    q, k, v, do = (t.to("cuda:0") for t in make_inputs(w))
    o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=True)
    a = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=True, dq_mode="atomic",
                 dq_split=0)
    b = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=True, dq_mode="atomic",
                 dq_split=0)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    ulp = 2.0 ** -7 * a[0].double().abs().max().item()
    assert (a[0].double() - b[0].double()).abs().max().item() <= ulp


MASK_CASES = [
    # (name, B, H, n, m, d, dv, dtype, mask, lq, lk, seed, layout)
    ("varlen_causal_d128", 3, 2, 700, 700, 128, 128, "bf16", "causal", [700, 513, 64],
     [700, 513, 64], 91, "bhsd"),
    ("varlen_br_cross_d64", 2, 2, 300, 900, 64, 64, "bf16", "causal_bottom_right", [300, 100],
     [900, 777], 92, "bhsd"),
    ("varlen_none_bshd_d128_dv64", 2, 3, 257, 600, 128, 64, "fp16", "none", [257, 1],
     [600, 300], 93, "bshd"),
    ("rows_without_keys_tl", 1, 2, 400, 300, 128, 128, "bf16", "causal_bottom_right", [400],
     [260], 94, "bhsd"),
    # top-left causal with more query than key blocks: the stored-dS
    # triangle indexes tiles past the dense layout's count
    ("causal_tl_600x300", 1, 2, 600, 300, 128, 128, "bf16", "causal", [600], [300], 99,
     "bhsd"),
    # causal with per-batch lengths in the [B, seq, H, dim] layout, fp16, d != dv
    ("varlen_causal_bshd_f16_d64_dv128", 2, 2, 520, 520, 64, 128, "fp16", "causal",
     [520, 300], [520, 300], 100, "bshd"),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: c[0])
def test_dq_modes_masks_and_layouts(case):
    name, B, H, n, m, d, dv, dtype, mask, lq, lk, seed, layout = case
    from test_gpu_masks import _inputs
    say(f"case {name}: B={B} H={H} n={n} m={m} d={d} dv={dv} {dtype} mask={mask} lq={lq} "
        f"lk={lk} layout={layout}")
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = _inputs(B, H, n, m, d, dv, dtype, seed, lq, lk)
    dev = "cuda:0"
    to_dev = (lambda t: t.transpose(1, 2).contiguous().to(dev)) if layout == "bshd" else \
        (lambda t: t.to(dev))
    back = (lambda t: t.transpose(1, 2)) if layout == "bshd" else (lambda t: t)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    sq = torch.tensor(lq, dtype=torch.int32, device=dev)
    sk = torch.tensor(lk, dtype=torch.int32, device=dev)
    o, lse = attn.fwd(qd, kd, vd, scale=scale, mask=mask, seqlens_q=sq, seqlens_k=sk,
                      layout=layout)
    ref = oracle.attn_bwd_masked(torch.nan_to_num(q), torch.nan_to_num(k), torch.nan_to_num(v),
                                 torch.nan_to_num(do), scale=scale, mask=mask, seqlens_q=lq,
                                 seqlens_k=lk)
    tol = TOL[dtype]
    nkb = (m + 255) // 256
    base = None
    modes = [("separate", None), ("auto", None), ("atomic", 0), ("atomic", 1), ("atomic", nkb)]
    if mask != "causal_bottom_right":
        modes.append(("stored_ds", None))
    for mode, split in modes:
        dq, dk, dvv = attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, mask=mask, seqlens_q=sq,
                               seqlens_k=sk, layout=layout, dq_mode=mode, dq_split=split)
        torch.cuda.synchronize()
        dq, dk, dvv = back(dq), back(dk), back(dvv)
        errs = {n_: rel_err(to64(t), ref[n_]) for n_, t in (("dq", dq), ("dk", dk), ("dv", dvv))}
        say(f"  {mode} split={split}: " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in errs.items()))
        for n_, e in errs.items():
            assert e <= tol, (name, mode, split, n_, e)
        # padded rows and keys are exact zeros in every mode
        for b in range(B):
            assert torch.all(dq[b, :, lq[b]:] == 0) and torch.all(dk[b, :, lk[b]:] == 0)
            assert torch.all(dvv[b, :, lk[b]:] == 0)
        if base is None:
            base = (dk.clone(), dvv.clone())
        else:
            assert torch.equal(dk, base[0]) and torch.equal(dvv, base[1]), (mode, split)


def test_stored_ds_refuses_a_moving_diagonal():
    """The stored-dS mode indexes dS tiles by a diagonal at j = i; with a
    bottom-right diagonal and per-batch lengths it is refused before
    anything runs, and ATTN_DQ_AUTO takes the separate pass there."""
    say("case stored_ds refusal, bottom-right with lengths")
    B, H, n, m, d = 2, 1, 200, 300, 64
    g = torch.Generator().manual_seed(95)
    q, k, v, do = (torch.randn(B, H, r, d, generator=g).to(torch.bfloat16).to("cuda:0")
                   for r in (n, m, m, n))
    sq = torch.tensor([200, 150], dtype=torch.int32, device="cuda:0")
    sk = torch.tensor([300, 250], dtype=torch.int32, device="cuda:0")
    o, lse = attn.fwd(q, k, v, mask="causal_bottom_right", seqlens_q=sq, seqlens_k=sk)
    with pytest.raises(attn.AttnError) as e:
        attn.bwd(q, k, v, o, do, lse, mask="causal_bottom_right", seqlens_q=sq,
                 seqlens_k=sk, dq_mode="stored_ds")
    assert e.value.status == attn.binding.ATTN_EUNSUPPORTED
    a = attn.bwd(q, k, v, o, do, lse, mask="causal_bottom_right", seqlens_q=sq, seqlens_k=sk)
    b = attn.bwd(q, k, v, o, do, lse, mask="causal_bottom_right", seqlens_q=sq, seqlens_k=sk,
                 dq_mode="separate")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_stored_ds_is_deterministic():
    """Two stored-dS calls give the same bits (no atomics in the mode)."""
    w = SHAPES[0]
    say(f"case stored_ds repeat {w.describe()}")
    q, k, v, do = (t.to("cuda:0") for t in make_inputs(w))
    o, lse = attn.fwd(q, k, v, scale=w.softmax_scale, causal=True)
    a = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=True, dq_mode="stored_ds")
    b = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=True, dq_mode="stored_ds")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)

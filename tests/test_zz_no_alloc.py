"""attn_bwd_ex_noalloc, the backward without a workspace argument (its
scratch is a static per-GPU array in the library), against attn_bwd_ex with
a workspace on the same inputs.

In the separate-pass dQ mode (what ATTN_DQ_AUTO picks) and the stored-dS
mode both entry points run the same kernels on the same data, so the
outputs must agree bit for bit.
In the atomic mode dQ is summed in an order the hardware chooses; there dK
and dV must still agree bit for bit and dQ within the bf16 bar
(max|err| / max|ref| <= 2e-2).  Each check makes two calls in a row, the
second on a smaller problem, so the second runs on scratch the first left
behind.
"""
import ctypes

import pytest
import torch

import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd import binding as B
from transformer_attn_bwd_amd.workloads import Workload, make_inputs

from gpu_util import TOL, rel_err, say, to64


def _w(name, Bt, H, n, m, d, dv, dtype, causal, seed):
    return Workload(name, Bt, H, n, m, d, dv, dtype, causal, seed)


def test_rejects_problems_beyond_the_static_scratch():
    """Host-side checks only: nothing is launched (the pointers are never
    dereferenced because the size check fails first)."""
    lib = B.load()
    fake = ctypes.c_void_p(1 << 20)
    # 64 * 32 * 4096 rows of D and LSE2 (8 bytes each) = 64 MiB > 16 MiB
    args = [fake] * 9 + [None, None, 64, 32, 4096, 4096, 128, 128, 0.088, B.ATTN_MASK_CAUSAL,
                         B.ATTN_LAYOUT_BHSD, B.ATTN_BF16]
    for mode in (B.ATTN_DQ_AUTO, B.ATTN_DQ_SEPARATE, B.ATTN_DQ_ATOMIC, B.ATTN_DQ_STORED_DS):
        st = lib.attn_bwd_ex_noalloc(*args, mode, None)
        assert st == B.ATTN_ESCRATCH, (mode, st)
    # the stored-dS tiles of 2 x 32 heads at 4096 (1.1 GB) exceed it as well,
    # while the automatic mode (the separate pass, 2 MiB of rows) fits
    small_ds = [fake] * 9 + [None, None, 2, 32, 4096, 4096, 128, 128, 0.088,
                             B.ATTN_MASK_CAUSAL, B.ATTN_LAYOUT_BHSD, B.ATTN_BF16]
    assert lib.attn_bwd_ex_noalloc(*small_ds, B.ATTN_DQ_STORED_DS, None) == B.ATTN_ESCRATCH
    # the atomic mode's accumulator: 64 heads * 4096 rows * 128 floats = 128 MiB
    small = [fake] * 9 + [None, None, 2, 32, 4096, 4096, 128, 128, 0.088, B.ATTN_MASK_CAUSAL,
                          B.ATTN_LAYOUT_BHSD, B.ATTN_BF16]
    assert lib.attn_bwd_ex_noalloc(*small, B.ATTN_DQ_ATOMIC, None) == B.ATTN_ESCRATCH
    # argument errors are reported before the size check
    bad = [fake] * 9 + [None, None, 2, 32, 4096, 4096, 130, 128, 0.088, B.ATTN_MASK_CAUSAL,
                        B.ATTN_LAYOUT_BHSD, B.ATTN_BF16]
    assert lib.attn_bwd_ex_noalloc(*bad, B.ATTN_DQ_AUTO, None) == B.ATTN_EUNSUPPORTED
    assert lib.attn_bwd_ex_noalloc(*small, 1 << 20, None) == B.ATTN_EUNSUPPORTED
    assert "scratch" in B.status_str(B.ATTN_ESCRATCH)


def _pair(w, dq_mode, dq_split=None, mask=None, seqlens=None, layout="bhsd"):
    """Outputs of the workspace entry point and of the no-allocation one."""
    dev = "cuda:0"
    q, k, v, do = (t.to(dev) for t in make_inputs(w))
    if layout == "bshd":
        q, k, v, do = (t.transpose(1, 2).contiguous() for t in (q, k, v, do))
    kw = dict(scale=w.softmax_scale, layout=layout)
    if mask is None:
        kw["causal"] = w.causal
    else:
        kw["mask"] = mask
    if seqlens is not None:
        kw["seqlens_q"] = torch.tensor(seqlens[0], dtype=torch.int32, device=dev)
        kw["seqlens_k"] = torch.tensor(seqlens[1], dtype=torch.int32, device=dev)
    o, lse = attn.fwd(q, k, v, **kw)
    ref = attn.bwd(q, k, v, o, do, lse, dq_mode=dq_mode, dq_split=dq_split, **kw)
    # outputs pre-filled with a pattern the library must overwrite
    got = tuple(torch.full_like(t, 7.0) for t in (q, k, v))
    attn.bwd_noalloc(q, k, v, o, do, lse, *got, dq_mode=dq_mode, dq_split=dq_split, **kw)
    torch.cuda.synchronize()
    return ref, got


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


SEQ = [
    (_w("noalloc_causal_1000_d128", 2, 4, 1000, 1000, 128, 128, "bf16", True, 61), "auto", None),
    (_w("noalloc_cross_300x700_d64", 1, 2, 300, 700, 64, 64, "bf16", False, 62), "auto", None),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_two_calls():
    for w, mode, split in SEQ:
        say(f"case noalloc {mode} {w.describe()}")
        ref, got = _pair(w, mode, split)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert _same_bits(a, b), (w.name, name, rel_err(to64(b), to64(a)))
    say("  bitwise equal on both calls")


@pytest.mark.gpu
def test_noalloc_separate_fp16_masked_bshd_two_calls():
    cases = [
        (_w("noalloc_f16_br_400x900_d128", 2, 3, 400, 900, 128, 128, "fp16", False, 63),
         "causal_bottom_right", ([400, 257], [900, 640]), "bshd"),
        (_w("noalloc_f16_causal_200_d96", 1, 2, 200, 200, 96, 96, "fp16", False, 64),
         "causal", ([200], [150]), "bhsd"),
    ]
    for w, mask, lens, layout in cases:
        say(f"case noalloc separate {mask} {layout} {w.describe()}")
        ref, got = _pair(w, "separate", None, mask, lens, layout)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert _same_bits(a, b), (w.name, name, rel_err(to64(b), to64(a)))
    say("  bitwise equal on both calls")


@pytest.mark.gpu
def test_noalloc_atomic_mode_two_calls():
    cases = [
        (_w("noalloc_atomic_causal_900_d128", 2, 4, 900, 900, 128, 128, "bf16", True, 65), 1),
        (_w("noalloc_atomic_causal_520_d64", 1, 3, 520, 520, 64, 64, "bf16", True, 66), 0),
    ]
    for w, split in cases:
        say(f"case noalloc atomic split {split} {w.describe()}")
        ref, got = _pair(w, "atomic", split)
        assert _same_bits(ref[1], got[1]) and _same_bits(ref[2], got[2]), w.name
        e = rel_err(to64(got[0]), to64(ref[0]))
        say(f"  dq vs workspace entry point {e:.3e}")
        assert e <= TOL["bf16"], (w.name, e)


@pytest.mark.gpu
def test_noalloc_stored_ds_two_calls():
    """The stored-dS mode keeps its dS tiles in the static scratch (1.5 MB
    and 0.4 MB here); deterministic, so bit for bit."""
    cases = [
        (_w("noalloc_stored_causal_600_d128", 1, 2, 600, 600, 128, 128, "bf16", True, 67), None),
        (_w("noalloc_stored_cross_200x500_d64", 1, 2, 200, 500, 64, 64, "bf16", False, 68), None),
    ]
    for w, split in cases:
        say(f"case noalloc stored_ds {w.describe()}")
        ref, got = _pair(w, "stored_ds", split)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert _same_bits(a, b), (w.name, name, rel_err(to64(b), to64(a)))
    say("  bitwise equal on both calls")

"""GPU parity: the HIP path against the float64 oracle, element by element,
on seeded inputs that span several tiles and end in ragged tails.

Bar (per output tensor): bf16 max|err| / max|ref| <= 2e-2; float16 2.5e-3;
float32 1e-5.  LSE is compared absolutely (16-bit paths 1e-3, float32 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd.workloads import WORKLOADS, Workload, make_inputs

from gpu_util import TOL, compare_full, oracle_full, rel_err, run_gpu, say, to64

pytestmark = pytest.mark.gpu


def _w(name, B, H, n, m, d, dv, dtype, causal, seed, qk_mult=1.0, scale=None):
    return Workload(name, B, H, n, m, d, dv, dtype, causal, seed, qk_mult, scale)


def test_fp32_head_64():
    """The single-head float32 workload, whole, against the oracle."""
    w = WORKLOADS["head_64_fp32"]
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    gpu = run_gpu(w, inputs)
    compare_full(w, gpu, oracle_full(w, inputs))


FP32_SHAPES = [
    _w("f32_ragged_causal", 2, 3, 77, 77, 48, 48, "fp32", True, 11),
    _w("f32_cross", 1, 2, 33, 130, 100, 20, "fp32", False, 12),
    _w("f32_d128", 1, 1, 65, 65, 128, 128, "fp32", True, 13),
    _w("f32_tiny", 1, 1, 1, 1, 1, 1, "fp32", False, 14),
]


@pytest.mark.parametrize("w", FP32_SHAPES, ids=lambda w: w.name)
def test_fp32_shapes(w):
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    compare_full(w, run_gpu(w, inputs), oracle_full(w, inputs))


BF16_SHAPES = [
    # several tiles in every direction, ragged tails, all three head-width pairs
    _w("bf16_causal_300_d64", 1, 2, 300, 300, 64, 64, "bf16", True, 21),
    _w("bf16_causal_257_d128", 2, 1, 257, 257, 128, 128, "bf16", True, 22),
    _w("bf16_cross_200x333_d128_dv64", 1, 2, 200, 333, 128, 64, "bf16", False, 23, 3.0),
    _w("bf16_cross_130x70_d128", 1, 1, 130, 70, 128, 128, "bf16", False, 24),
    _w("bf16_noncausal_129x129_d64", 1, 3, 129, 129, 64, 64, "bf16", False, 25),
    _w("bf16_causal_384_d128", 1, 1, 384, 384, 128, 128, "bf16", True, 26),
    _w("bf16_single_key", 1, 1, 5, 1, 64, 64, "bf16", False, 27),
    _w("bf16_single_row", 1, 1, 1, 1, 128, 64, "bf16", True, 28),
    _w("bf16_cross_1x500_d128", 1, 1, 1, 500, 128, 128, "bf16", False, 29),
    _w("bf16_stress_x30", 1, 1, 70, 90, 128, 64, "bf16", False, 30, 30.0 ** 0.5),
    # several 256-row workgroups in each direction, ragged against 256, 64, 32
    _w("bf16_causal_700_d128", 1, 2, 700, 700, 128, 128, "bf16", True, 31),
    _w("bf16_cross_600x900_d128_dv64", 1, 1, 600, 900, 128, 64, "bf16", False, 32),
    _w("bf16_causal_520_d64", 2, 1, 520, 520, 64, 64, "bf16", True, 33),
    # many heads: grids of 512 workgroups and more, several per compute unit
    _w("bf16_4wave_causal_300_d128", 4, 64, 300, 300, 128, 128, "bf16", True, 36),
    _w("bf16_4wave_cross_260x530_d64", 2, 128, 260, 530, 64, 64, "bf16", False, 37),
    # scale signs the kernels treat specially: negative (the forward negates
    # Q) and zero (uniform P over the visible keys)
    _w("bf16_negative_scale", 1, 1, 100, 150, 128, 128, "bf16", False, 34, 1.0, -0.1),
    _w("bf16_zero_scale_causal", 1, 1, 90, 90, 64, 64, "bf16", True, 35, 1.0, 0.0),
]


@pytest.mark.parametrize("w", BF16_SHAPES, ids=lambda w: w.name)
def test_bf16_shapes(w):
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    compare_full(w, run_gpu(w, inputs), oracle_full(w, inputs))


FP16_SHAPES = [
    # the same kernels instantiated for IEEE half: every head-width pair,
    # ragged tails across several workgroups, both masks, and the scale
    # signs the forward treats specially
    _w("f16_causal_700_d128", 1, 2, 700, 700, 128, 128, "fp16", True, 51),
    _w("f16_cross_600x900_d128_dv64", 1, 1, 600, 900, 128, 64, "fp16", False, 52, 3.0),
    _w("f16_causal_300_d64", 2, 1, 300, 300, 64, 64, "fp16", True, 53),
    _w("f16_noncausal_129x333_d64", 1, 3, 129, 333, 64, 64, "fp16", False, 54),
    _w("f16_single_row", 1, 1, 1, 1, 128, 64, "fp16", True, 55),
    _w("f16_stress_x30", 1, 1, 70, 90, 128, 64, "fp16", False, 56, 30.0 ** 0.5),
    _w("f16_negative_scale", 1, 1, 100, 150, 128, 128, "fp16", False, 57, 1.0, -0.1),
    _w("f16_zero_scale_causal", 1, 1, 90, 90, 64, 64, "fp16", True, 58, 1.0, 0.0),
]


@pytest.mark.parametrize("w", FP16_SHAPES, ids=lambda w: w.name)
def test_fp16_shapes(w):
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    compare_full(w, run_gpu(w, inputs), oracle_full(w, inputs))


WIDTH_SHAPES = [
    # head widths other than 64 and 128 (multiples of 8 up to 128): the
    # kernels pad them with zero columns to 64- or 128-wide tiles
    _w("bf16_d32_causal", 1, 2, 300, 300, 32, 32, "bf16", True, 61),
    _w("bf16_d96_cross", 1, 2, 200, 333, 96, 96, "bf16", False, 62),
    _w("bf16_d80_causal", 2, 1, 257, 257, 80, 80, "bf16", True, 63),
    _w("bf16_d64_dv128", 1, 2, 300, 300, 64, 128, "bf16", True, 64),
    _w("bf16_d8_dv8", 1, 1, 130, 70, 8, 8, "bf16", False, 65),
    _w("bf16_d128_dv32", 1, 2, 190, 190, 128, 32, "bf16", True, 66),
    _w("bf16_d40_dv72", 1, 1, 100, 520, 40, 72, "bf16", False, 67),
    _w("bf16_d112_dv120", 1, 1, 333, 333, 112, 120, "bf16", True, 68),
    _w("f16_d96_causal", 1, 2, 400, 400, 96, 96, "fp16", True, 69),
    _w("f16_d48_dv128", 1, 1, 150, 300, 48, 128, "fp16", False, 70, 3.0),
]


@pytest.mark.parametrize("w", WIDTH_SHAPES, ids=lambda w: w.name)
def test_head_widths(w):
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    compare_full(w, run_gpu(w, inputs), oracle_full(w, inputs))


def test_fp16_and_bf16_agree_on_exact_inputs():
    """Inputs that both 16-bit types hold exactly (small integers times
    powers of two) give the two instantiations the same problem; their
    results differ only by the rounding of P, dS and the outputs."""
    w = _w("both16", 1, 2, 200, 200, 128, 128, "bf16", True, 59)
    g = torch.Generator().manual_seed(59)
    base = [torch.randint(-8, 9, s, generator=g).float() / 8
            for s in ((1, 2, 200, 128),) * 4]
    ref = oracle_full(w, base)
    for dt, name in ((torch.bfloat16, "bf16"), (torch.float16, "fp16")):
        ins = [t.to(dt) for t in base]
        assert all(torch.equal(a.float(), b) for a, b in zip(ins, base))
        out = run_gpu(w.with_(dtype=name), ins)
        for key in ("o", "dq", "dk", "dv"):
            e = rel_err(to64(out[key]), ref[key])
            say(f"  {name} {key} {e:.3e}")
            assert e <= TOL[name], (name, key, e)


@pytest.mark.parametrize("w", [BF16_SHAPES[0], BF16_SHAPES[2], BF16_SHAPES[5]], ids=lambda w: w.name)
def test_bwd_alone_from_oracle_forward(w):
    """The backward fed the oracle's O (rounded to bf16) and LSE, so that its
    error is measured apart from the forward kernel's."""
    say(f"case bwd-only {w.describe()}")
    inputs = make_inputs(w, "cuda:0")
    ref = oracle_full(w, inputs)
    q, k, v, do = inputs
    o = torch.from_numpy(ref["o"]).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(ref["lse"]).float().cuda()
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal)
    torch.cuda.synchronize()
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        e = rel_err(to64(got), ref[name])
        say(f"  {name} {e:.3e}")
        assert e <= TOL["bf16"], (name, e)


def test_causal_1k_d64_whole_heads():
    """The B=4, H=16, n=m=1024, d=64 causal workload: four heads compared
    whole (every element) against the oracle."""
    w = WORKLOADS["causal_1k_d64"]
    say(f"case {w.describe()}")
    inputs = make_inputs(w)
    gpu = run_gpu(w, inputs)
    heads = [(0, 0), (w.B - 1, w.H - 1), (1, 7), (2, 3)]
    for (b, h) in heads:
        sub = [t[b:b + 1, h:h + 1] for t in inputs]
        ref = oracle.attn_bwd(*(to64(t) for t in sub), scale=w.softmax_scale, causal=w.causal)
        for name in ("o", "dq", "dk", "dv"):
            e = rel_err(to64(gpu[name][b:b + 1, h:h + 1]), ref[name])
            assert e <= TOL["bf16"], ((b, h), name, e)
        assert np.max(np.abs(to64(gpu["lse"][b:b + 1, h:h + 1]) - ref["lse"])) <= 1e-3
    say("  4 heads ok")


def test_determinism_bitwise():
    """No atomics: repeated backward calls give identical bits."""
    w = _w("det", 2, 2, 320, 320, 128, 128, "bf16", True, 40)
    inputs = make_inputs(w, "cuda:0")
    q, k, v, do = inputs
    o, lse = attn.fwd(q, k, v, causal=True)
    a = attn.bwd(q, k, v, o, do, lse, causal=True)
    b = attn.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_n_zero_gives_zero_key_gradients():
    """No queries: dK and dV are empty sums, i.e. zero."""
    dev = "cuda:0"
    for dtype in (torch.bfloat16, torch.float16, torch.float32):
        q = torch.empty(1, 2, 0, 64, dtype=dtype, device=dev)
        k = torch.randn(1, 2, 70, 64, device=dev).to(dtype)
        v = torch.randn(1, 2, 70, 64, device=dev).to(dtype)
        o = torch.empty(1, 2, 0, 64, dtype=dtype, device=dev)
        lse = torch.empty(1, 2, 0, dtype=torch.float32, device=dev)
        dk = torch.full_like(k, 7.0)
        dv = torch.full_like(v, 7.0)
        attn.bwd(q, k, v, o, o, lse, dk=dk, dv=dv)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def test_error_leaves_outputs_untouched():
    dev = "cuda:0"
    w = _w("err", 1, 1, 64, 64, 64, 64, "bf16", False, 41)
    q, k, v, do = make_inputs(w, dev)
    o, lse = attn.fwd(q, k, v)
    dq = torch.full_like(q, 3.0)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(attn.AttnError) as ei:
        attn.bwd(q, k, v, o, do, lse, workspace=small, dq=dq)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(dq == 3.0)


STAGE_CASES = [
    # (name, B, H, n, m, d, dv, dtype, mask, lengths q, lengths k, layout, seed)
    ("bf16_causal_d128", 2, 2, 300, 300, 128, 128, torch.bfloat16, "causal", None, None,
     "bhsd", 42),
    ("fp16_causal_d64", 2, 3, 257, 257, 64, 64, torch.float16, "causal", None, None, "bhsd", 44),
    ("bf16_cross_d128_dv64", 1, 2, 200, 333, 128, 64, torch.bfloat16, "none", None, None,
     "bhsd", 45),
    ("bf16_varlen_br_d40_dv72_bshd", 3, 2, 300, 260, 40, 72, torch.bfloat16,
     "causal_bottom_right", [300, 129, 5], [260, 200, 33], "bshd", 46),
]


@pytest.mark.parametrize("case", STAGE_CASES, ids=lambda c: c[0])
def test_stages_compose_to_the_whole_backward(case):
    """Running the preprocess, dK/dV and dQ kernels as three calls (the
    timing flags) gives the bits of one call, in which the dQ pass does
    the preprocess for its rows: the workspace (LSE in base 2 and D for
    every padded row) and dQ, dK, dV are equal bit for bit.  The cases
    cover both reduction shapes of D (64- and 128-wide tiles), a width
    short of its tile, lengths, padded rows and the [B, seq, H, dim]
    layout."""
    name, B, H, n, m, d, dv, dt, mask, lq, lk, layout, seed = case
    say(f"case stages {name}")
    dev = "cuda:0"
    g = torch.Generator().manual_seed(seed)
    shp = (lambda rows, w: (B, rows, H, w)) if layout == "bshd" else \
        (lambda rows, w: (B, H, rows, w))
    q, k = (torch.randn(shp(r_, d), generator=g).to(dt).to(dev) for r_ in (n, m))
    v = torch.randn(shp(m, dv), generator=g).to(dt).to(dev)
    do = torch.randn(shp(n, dv), generator=g).to(dt).to(dev)
    sq = torch.tensor(lq, dtype=torch.int32, device=dev) if lq else None
    sk = torch.tensor(lk, dtype=torch.int32, device=dev) if lk else None
    kw = dict(mask=mask, seqlens_q=sq, seqlens_k=sk, layout=layout)
    o, lse = attn.fwd(q, k, v, **kw)
    nbytes = attn.bwd_workspace_bytes(B, H, n, m, d, dv, dt)
    n_pad = (n + 127) // 128 * 128
    used = 2 * B * H * n_pad           # floats: LSE2 then D
    ws1 = torch.full((nbytes,), 7, dtype=torch.uint8, device=dev)
    ws2 = torch.full((nbytes,), 9, dtype=torch.uint8, device=dev)
    whole = attn.bwd(q, k, v, o, do, lse, workspace=ws1, **kw)
    parts = [torch.full_like(t, 5.0) for t in (q, k, v)]
    for stage in ("preprocess", "dkdv", "dq"):
        attn.bwd(q, k, v, o, do, lse, workspace=ws2, dq=parts[0], dk=parts[1], dv=parts[2],
                 stages=[stage], **kw)
    torch.cuda.synchronize()
    assert torch.equal(ws1[:4 * used], ws2[:4 * used])
    for a_, b_ in zip(whole, parts):
        assert torch.equal(a_, b_)


def test_determinism_fp16_masked_bshd():
    """No atomics anywhere: repeated calls with lengths, the bottom-right
    mask and the [B, seq, H, dim] layout give identical bits."""
    dev = "cuda:0"
    g = torch.Generator().manual_seed(43)
    q, k, v, do = (torch.randn((3, 200, 2, 64), generator=g).to(torch.float16).to(dev)
                   for _ in range(4))
    sq = torch.tensor([200, 150, 7], dtype=torch.int32, device=dev)
    sk = torch.tensor([180, 200, 30], dtype=torch.int32, device=dev)
    kw = dict(mask="causal_bottom_right", seqlens_q=sq, seqlens_k=sk, layout="bshd")
    o1, l1 = attn.fwd(q, k, v, **kw)
    o2, l2 = attn.fwd(q, k, v, **kw)
    a = attn.bwd(q, k, v, o1, do, l1, **kw)
    b = attn.bwd(q, k, v, o1, do, l1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_side_stream_matches_default_stream():
    """Work is enqueued on the caller's current stream: the same call on a
    side stream (default priority) gives the same bits once synchronised."""
    w = _w("stream", 1, 2, 260, 260, 64, 64, "bf16", True, 44)
    q, k, v, do = make_inputs(w, "cuda:0")
    o, lse = attn.fwd(q, k, v, causal=True)
    ref = attn.bwd(q, k, v, o, do, lse, causal=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, lse2 = attn.fwd(q, k, v, causal=True)
        got = attn.bwd(q, k, v, o2, do, lse2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_hip_graph_capture_and_replay():
    """The entry points launch kernels only (no allocation, no memset, no
    synchronisation), so a forward + backward can be captured in a HIP
    graph; every replay, with eager work and synchronisations between
    them, reproduces the eager result bit for bit."""
    w = _w("graph", 2, 2, 300, 300, 128, 128, "bf16", True, 45)
    dev = "cuda:0"
    q, k, v, do = make_inputs(w, dev)
    ws = torch.empty(attn.bwd_workspace_bytes(2, 2, 300, 300, 128, 128), dtype=torch.uint8,
                     device=dev)
    o, lse = torch.empty_like(q), torch.empty(2, 2, 300, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        attn.fwd(q, k, v, causal=True, out=o, lse=lse)
        attn.bwd(q, k, v, o, do, lse, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(0.5)                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((o, lse, dq, dk, dv), ref):
            assert torch.equal(a, b)

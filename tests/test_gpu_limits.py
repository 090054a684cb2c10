"""GPU parity at the size limits of the C ABI.

The 16-bit kernels address one head's rows through 32-bit buffer offsets,
so the library accepts a [B, seq, H, dim] problem only while one tensor's
rows span at most 2^30 bytes.  This test runs the largest such problem (n
= m = 65536 rows, H = 64 heads of width 128, bf16: each tensor exactly
2^30 bytes), causal, and compares sampled query rows (O, LSE, dQ) and
key rows (dK, dV) of two heads with the oracle's sampled routines
("Attention Backpropagation: Step by step derivation", sections Gradient
of S and Gradient of Q and K; eulerpad "Attention backward" P2-P8).  One
row more is rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd import binding

from gpu_util import TOL, rel_err, say, to64

pytestmark = pytest.mark.gpu


def test_bshd_byte_limit_sampled():
    B, H, n, d = 1, 64, 65536, 128
    assert n * H * d * 2 == 1 << 30
    dev = "cuda:0"
    say(f"case bshd byte limit: B={B} n=m={n} H={H} d=dv={d} bf16 causal")
    g = torch.Generator(device=dev).manual_seed(160)
    # seeded N(0,1) inputs drawn on the device (8 GiB of host float64 would
    # be needed to draw them on the CPU); the sampled heads are copied back
    q, k, v, do = (torch.randn((B, n, H, d), generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(4))
    scale = 1.0 / np.sqrt(d)
    o, lse = attn.fwd(q, k, v, scale=scale, mask="causal", layout="bshd")
    dq, dk, dvv = attn.bwd(q, k, v, o, do, lse, scale=scale, mask="causal", layout="bshd")
    torch.cuda.synchronize()

    rng = np.random.default_rng(161)
    worst = {}
    for h in (0, H - 1):
        Q, K, V, dO = (to64(t[0, :, h]) for t in (q, k, v, do))
        # The bar is per tensor, max|err| / max|ref|: the samples include the
        # first 64 rows and keys, where dQ (rows that see few keys) and dK,
        # dV (keys that every row sees) are largest, so that the sampled
        # max|ref| stands for the tensor's.
        rows = sorted({*range(64), n // 2, n - 1, *rng.choice(n, 6, replace=False).tolist()})
        cols = sorted({*range(64), n // 2, n - 2, n - 1,
                       *rng.choice(n, 6, replace=False).tolist()})
        r = oracle.attn_rows(Q, K, V, dO, rows, scale=scale, causal=True)
        c = oracle.attn_cols(Q, K, V, dO, cols, scale=scale, causal=True)
        errs = {
            "o": rel_err(to64(o[0, rows, h]), r["o"]),
            "dq": rel_err(to64(dq[0, rows, h]), r["dq"]),
            "dk": rel_err(to64(dk[0, cols, h]), c["dk"]),
            "dv": rel_err(to64(dvv[0, cols, h]), c["dv"]),
            "lse_abs": float(np.max(np.abs(to64(lse[0, h, rows]) - r["lse"]))),
        }
        for key, val in errs.items():
            worst[key] = max(worst.get(key, 0.0), val)
    say("  worst " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in worst.items()))
    for key in ("o", "dq", "dk", "dv"):
        assert worst[key] <= TOL["bf16"], (key, worst[key])
    assert worst["lse_abs"] <= 1e-3

    # one row more: every tensor passes 2^30 bytes, and the call is refused
    del q, k, v, do, o, lse, dq, dk, dvv
    torch.cuda.empty_cache()
    n1 = n + 1
    t = torch.zeros((B, n1, H, d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.AttnError) as err:
        attn.fwd(t, t, t, scale=scale, mask="causal", layout="bshd")
    assert err.value.status == binding.ATTN_EUNSUPPORTED

"""Seeded synthetic inputs for attention forward/backward.

This module holds the workload definitions and the random-number recipe and
nothing else: no attention arithmetic.  Both the HIP path's tests and the
oracle draw their inputs from here, so that each side sees identical values.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws
i.i.d. standard normal float32 values with ``torch.randn`` in the order
Q [B,H,n,d], K [B,H,m,d], V [B,H,m,dv], dO [B,H,n,dv]; Q and K are then
multiplied by ``qk_mult`` (3.0 for the cross-attention stress case, so raw
logits reach about +-100) and every tensor is rounded to the workload's
dtype (round to nearest even for bfloat16 and float16).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    m: int
    d: int
    dv: int
    dtype: str          # "fp32", "bf16" or "fp16"
    causal: bool
    seed: int
    qk_mult: float = 1.0
    scale: float | None = None   # None means 1/sqrt(d)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "n": self.n, "m": self.m,
                "d": self.d, "dv": self.dv, "dtype": self.dtype, "causal": self.causal,
                "seed": self.seed, "qk_mult": self.qk_mult, "scale": self.softmax_scale}


# The five workloads: shapes, dtypes, masks and seeds of the method's test
# configurations.  The headline throughput workload is "causal_4k_d128".
WORKLOADS = {
    "head_64_fp32": Workload("head_64_fp32", 1, 1, 64, 64, 64, 64, "fp32", False, 0),
    "causal_1k_d64": Workload("causal_1k_d64", 4, 16, 1024, 1024, 64, 64, "bf16", True, 1),
    "causal_4k_d128": Workload("causal_4k_d128", 2, 32, 4096, 4096, 128, 128, "bf16", True, 2),
    "causal_16k_d128": Workload("causal_16k_d128", 1, 32, 16384, 16384, 128, 128, "bf16", True, 3),
    "cross_512x2048_d128_dv64": Workload("cross_512x2048_d128_dv64", 8, 16, 512, 2048, 128, 64,
                                         "bf16", False, 4, qk_mult=3.0),
    # the headline shape with IEEE half inputs (same seed, rounded to float16)
    "causal_4k_d128_fp16": Workload("causal_4k_d128_fp16", 2, 32, 4096, 4096, 128, 128, "fp16",
                                    True, 2),
}
HEADLINE = "causal_4k_d128"


def make_inputs(w: Workload, device: str | torch.device = "cpu"):
    """(q, k, v, do) as contiguous [B,H,seq,dim] tensors of w's dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    q = torch.randn((w.B, w.H, w.n, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.H, w.m, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.H, w.m, w.dv), generator=g, dtype=torch.float32)
    do = torch.randn((w.B, w.H, w.n, w.dv), generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q.mul_(w.qk_mult)
        k.mul_(w.qk_mult)
    dt = w.torch_dtype
    return tuple(t.to(dt).contiguous().to(device) for t in (q, k, v, do))

"""Scaled dot-product attention backward for AMD Instinct MI355X (gfx950).

The computation lives in libattn.so (hand-written HIP kernels behind the C
ABI declared in include/attn.h); this package is its ctypes binding plus the
seeded synthetic workloads used by the tests and the benchmark.
"""
from .binding import (AttnError, LIB_PATH, bwd, bwd_noalloc, bwd_workspace_bytes, fwd,  # noqa: F401
                      in_proj_bwd, load, out_proj_bwd, status_str)

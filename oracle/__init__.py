"""Float64 CPU oracle for scaled dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.
It shares no code with the HIP path.  The arithmetic lives in
``attn_oracle.c`` (plain loops in float64, the row-by-row definition of the
gradients); this module only builds that file with gcc and marshals numpy
arrays through ctypes.

Every function takes and returns float64 numpy arrays laid out as
[B, H, rows, cols] (the [batch, heads, seq, head_dim] shape of the
step-by-step derivation's "Forward Pass").  The scale defaults to 1/sqrt(d)
with d the width of Q (mlgrind "Forward").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

# Known-wrong variants (negative controls); values match the C enum.
EXACT = 0
WRONG_DS_NO_CORRECTION = 1
WRONG_DS_DIAG_ONLY = 2
WRONG_DV_NO_TRANSPOSE = 3
WRONG_FLAT_JACOBIAN = 4
WRONG_DROP_SCALE = 5
WRONG_MASK_AFTER = 6
WRONG_VARIANTS = {
    "ds_no_correction": WRONG_DS_NO_CORRECTION,
    "ds_diag_only": WRONG_DS_DIAG_ONLY,
    "dv_no_transpose": WRONG_DV_NO_TRANSPOSE,
    "flat_jacobian": WRONG_FLAT_JACOBIAN,
    "drop_scale": WRONG_DROP_SCALE,
    "mask_after_softmax": WRONG_MASK_AFTER,
}


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so with gcc and OpenMP."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_long)
    L, D, I = ctypes.c_long, ctypes.c_double, ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, L, D, I]
    lib.oracle_attn_fwd.restype = I
    lib.oracle_attn_bwd.argtypes = [dp] * 12 + [L] * 6 + [D, I, I]
    lib.oracle_attn_bwd.restype = I
    lib.oracle_attn_bwd_masked.argtypes = [dp] * 10 + [L] * 6 + [D, I, lp, lp]
    lib.oracle_attn_bwd_masked.restype = I
    lib.oracle_attn_rows.argtypes = [dp, dp, dp, dp, L, L, L, L, D, I, L, lp, L, dp, dp, dp, dp]
    lib.oracle_attn_rows.restype = I
    lib.oracle_attn_cols.argtypes = [dp, dp, dp, dp, L, L, L, L, D, I, L, lp, L, dp, dp]
    lib.oracle_attn_cols.restype = I
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Contiguous float64 copy of an array-like (torch tensors included)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as4d(x: np.ndarray) -> np.ndarray:
    if x.ndim == 2:
        return x[None, None]
    if x.ndim == 3:
        return x[:, None]
    if x.ndim != 4:
        raise ValueError(f"expected a 2-, 3- or 4-d array, got shape {x.shape}")
    return x


def _dims(q, k, v):
    B, H, n, d = q.shape
    Bk, Hk, m, dk = k.shape
    Bv, Hv, mv, dv = v.shape
    if (Bk, Hk, dk) != (B, H, d) or (Bv, Hv, mv) != (B, H, m):
        raise ValueError(f"inconsistent shapes q{q.shape} k{k.shape} v{v.shape}")
    return B, H, n, m, d, dv


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def attn_fwd(q, k, v, scale=None, causal=False):
    """O [B,H,n,dv] and LSE [B,H,n] (natural log) in float64."""
    q0 = _f64(q)
    squeeze = q0.ndim
    q, k, v = _as4d(q0), _as4d(_f64(k)), _as4d(_f64(v))
    B, H, n, m, d, dv = _dims(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((B, H, n, dv))
    lse = np.zeros((B, H, n))
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 B, H, n, m, d, dv, float(scale), int(bool(causal)))
    if rc:
        raise ValueError("oracle_attn_fwd: invalid sizes (m must be > 0; causal needs n == m)")
    if squeeze == 2:
        return o[0, 0], lse[0, 0]
    if squeeze == 3:
        return o[:, 0], lse[:, 0]
    return o, lse


def attn_bwd(q, k, v, dout, scale=None, causal=False, variant=EXACT, want_ds=False):
    """Gradients by the definition, recomputing P.

    Returns a dict with dq, dk, dv, D (rowsum(dP o P)), D_alt
    (rowsum(dO o O)), o, lse and, if want_ds, ds [B,H,n,m].
    """
    q0 = _f64(q)
    ndim = q0.ndim
    q, k, v, do = _as4d(q0), _as4d(_f64(k)), _as4d(_f64(v)), _as4d(_f64(dout))
    B, H, n, m, d, dv = _dims(q, k, v)
    if do.shape != (B, H, n, dv):
        raise ValueError(f"dout shape {do.shape} != {(B, H, n, dv)}")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = {
        "dq": np.zeros((B, H, n, d)), "dk": np.zeros((B, H, m, d)),
        "dv": np.zeros((B, H, m, dv)), "D": np.zeros((B, H, n)),
        "D_alt": np.zeros((B, H, n)), "o": np.zeros((B, H, n, dv)),
        "lse": np.zeros((B, H, n)),
    }
    ds = np.zeros((B, H, n, m)) if want_ds else None
    rc = _load().oracle_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["D"]), _ptr(out["D_alt"]), _ptr(out["o"]),
        _ptr(out["lse"]), _ptr(ds) if ds is not None else None,
        B, H, n, m, d, dv, float(scale), int(bool(causal)), int(variant))
    if rc:
        raise ValueError("oracle_attn_bwd: invalid sizes or variant")
    if want_ds:
        out["ds"] = ds
    if ndim == 2:
        out = {key: val[0, 0] for key, val in out.items()}
    elif ndim == 3:
        out = {key: val[:, 0] for key, val in out.items()}
    return out


def attn_rows(q, k, v, dout, rows, scale=None, causal=False, causal_offset=0):
    """One head: O, LSE, D and dQ for the listed query rows only.  Under the
    causal mask key j is visible from row i when j <= i + causal_offset."""
    q, k, v, do = (_f64(t) for t in (q, k, v, dout))
    n, d = q.shape
    m, dv = v.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    r = len(rows)
    o = np.zeros((r, dv)); lse = np.zeros(r); D = np.zeros(r); dq = np.zeros((r, d))
    rc = _load().oracle_attn_rows(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), n, m, d, dv, float(scale), int(bool(causal)),
        int(causal_offset), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), r, _ptr(o),
        _ptr(lse), _ptr(D), _ptr(dq))
    if rc:
        raise ValueError("oracle_attn_rows: invalid arguments")
    return {"o": o, "lse": lse, "D": D, "dq": dq}


def attn_cols(q, k, v, dout, cols, scale=None, causal=False, causal_offset=0):
    """One head: dK and dV for the listed key rows only (causal mask as in
    attn_rows)."""
    q, k, v, do = (_f64(t) for t in (q, k, v, dout))
    n, d = q.shape
    m, dv = v.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    c = len(cols)
    dk = np.zeros((c, d)); dvv = np.zeros((c, dv))
    rc = _load().oracle_attn_cols(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), n, m, d, dv, float(scale), int(bool(causal)),
        int(causal_offset), cols.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), c, _ptr(dk),
        _ptr(dvv))
    if rc:
        raise ValueError("oracle_attn_cols: invalid arguments")
    return {"dk": dk, "dv": dvv}


MASKS = {"none": 0, "causal": 1, "causal_bottom_right": 2}


def attn_bwd_masked(q, k, v, dout, scale=None, mask="none", seqlens_q=None, seqlens_k=None):
    """Forward and backward with per-batch lengths and a mask mode.

    ``mask``: "none", "causal" (key j visible from row i when j <= i) or
    "causal_bottom_right" (j <= i + nk[b] - nq[b]).  ``seqlens_q`` and
    ``seqlens_k`` (length B, or None for n and m) give the rows of each
    batch element that take part; the rest is padding.  Rows that see no
    key, and padded rows, get O = 0, LSE = -inf, D = 0, dQ = 0; padded keys
    get dK = dV = 0.  Returns a dict with o, lse, D, dq, dk, dv as
    [B,H,...] float64 arrays.
    """
    q, k, v, do = (_as4d(_f64(t)) for t in (q, k, v, dout))
    B, H, n, m, d, dv = _dims(q, k, v)
    if do.shape != (B, H, n, dv):
        raise ValueError(f"dout shape {do.shape} != {(B, H, n, dv)}")
    if scale is None:
        scale = 1.0 / np.sqrt(d)

    def lens(x):
        if x is None:
            return None
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int64).reshape(-1))
        if a.shape != (B,):
            raise ValueError(f"sequence lengths need shape ({B},), got {a.shape}")
        return a

    lq, lk = lens(seqlens_q), lens(seqlens_k)
    out = {
        "dq": np.zeros((B, H, n, d)), "dk": np.zeros((B, H, m, d)),
        "dv": np.zeros((B, H, m, dv)), "D": np.zeros((B, H, n)),
        "o": np.zeros((B, H, n, dv)), "lse": np.zeros((B, H, n)),
    }
    lp = ctypes.POINTER(ctypes.c_long)
    rc = _load().oracle_attn_bwd_masked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["D"]), _ptr(out["o"]), _ptr(out["lse"]),
        B, H, n, m, d, dv, float(scale), MASKS[mask],
        lq.ctypes.data_as(lp) if lq is not None else None,
        lk.ctypes.data_as(lp) if lk is not None else None)
    if rc:
        raise ValueError("oracle_attn_bwd_masked: invalid sizes or mask")
    return out


# ---------------------------------------------------------------- projections
#
# The layer around attention (eulerpad "Attention backward" Problems 7 and
# 10; datatweets "Step 4: Back to the Parameters and Input"): for tokens
# t = 1..T (batch and sequence flattened), X [T, d_model], Q = X W_Q,
# K = X W_K, V = X W_V with W_Q, W_K [d_model, H d] and W_V [d_model, H dv]
# holding the heads side by side (columns (h-1) d + 1 .. h d belong to head
# h), and Y = O_cat W_O with O_cat [T, H dv] the heads' outputs side by side
# and W_O [H dv, d_model].  Plain float64 matrix products of the stated
# formulas; the weights' gradients sum over every token.


def out_proj_bwd(o_cat, g, w_o):
    """Problem 10: for Y = O_cat W_O and G = dL/dY, dW_O = O_cat^T G and
    dL/dO_cat = G W_O^T (whose column block h is head h's dO).
    o_cat [T, H dv], g [T, d_model], w_o [H dv, d_model]."""
    o_cat, g, w_o = _f64(o_cat), _f64(g), _f64(w_o)
    return {"dw_o": o_cat.T @ g, "do_cat": g @ w_o.T}


def in_proj_bwd(x, w_q, w_k, w_v, dq_cat, dk_cat, dv_cat):
    """Problem 7: dW_Q = X^T dQ, dW_K = X^T dK, dW_V = X^T dV and
    dX = dQ W_Q^T + dK W_K^T + dV W_V^T (X feeds all three projections, so
    the three paths add).  x [T, d_model]; dq_cat, dk_cat [T, H d];
    dv_cat [T, H dv]."""
    x, w_q, w_k, w_v = (_f64(t) for t in (x, w_q, w_k, w_v))
    dq, dk, dv = (_f64(t) for t in (dq_cat, dk_cat, dv_cat))
    return {"dw_q": x.T @ dq, "dw_k": x.T @ dk, "dw_v": x.T @ dv,
            "dx": dq @ w_q.T + dk @ w_k.T + dv @ w_v.T}

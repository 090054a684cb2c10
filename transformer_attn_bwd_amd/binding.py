"""Thin ctypes binding over libattn.so.

Argument marshalling only: PyTorch supplies device memory and the current
HIP stream; every step of the computation runs in the library's kernels.
If the library has not been built the first call raises; there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

# Values of include/attn.h.
ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2
_DTYPE_CODES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}
(ATTN_OK, ATTN_EINVAL, ATTN_ECAUSAL_SHAPE, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_EHIP,
 ATTN_ESCRATCH) = range(7)
NOALLOC_SCRATCH_BYTES = 16 << 20
ATTN_DQ_AUTO, ATTN_DQ_ATOMIC, ATTN_DQ_SEPARATE, ATTN_DQ_STORED_DS = 0, 1, 2, 3
DQ_SPLIT_SHIFT, DQ_SPLIT_MAX = 12, 255
ATTN_MASK_NONE, ATTN_MASK_CAUSAL, ATTN_MASK_CAUSAL_BOTTOM_RIGHT = 0, 1, 2
MASKS = {"none": ATTN_MASK_NONE, "causal": ATTN_MASK_CAUSAL,
         "causal_bottom_right": ATTN_MASK_CAUSAL_BOTTOM_RIGHT}
ATTN_LAYOUT_BHSD, ATTN_LAYOUT_BSHD = 0, 1
LAYOUTS = {"bhsd": ATTN_LAYOUT_BHSD, "bshd": ATTN_LAYOUT_BSHD}
ATTN_STAGE_PREPROCESS, ATTN_STAGE_DKDV, ATTN_STAGE_DQ = 1 << 8, 1 << 9, 1 << 10
DQ_MODES = {"auto": ATTN_DQ_AUTO, "atomic": ATTN_DQ_ATOMIC, "separate": ATTN_DQ_SEPARATE,
            "stored_ds": ATTN_DQ_STORED_DS}
STAGES = {"preprocess": ATTN_STAGE_PREPROCESS, "dkdv": ATTN_STAGE_DKDV, "dq": ATTN_STAGE_DQ}

EXPORTED = ("attn_fwd", "attn_fwd_ex", "attn_bwd", "attn_bwd_ex", "attn_bwd_workspace_bytes",
            "attn_bwd_workspace_bytes_ex", "attn_bwd_ex_noalloc",
            "attn_out_proj_bwd", "attn_in_proj_bwd", "attn_status_str", "attn_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def load():
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m transformer_attn_bwd_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, I, I, I, I, I, I, F, I, I, vp]
    lib.attn_fwd.restype = I
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.attn_bwd_workspace_bytes.restype = Z
    lib.attn_bwd_workspace_bytes_ex.argtypes = [I] * 9
    lib.attn_bwd_workspace_bytes_ex.restype = Z
    lib.attn_bwd.argtypes = [vp] * 9 + [I] * 6 + [F, I, I, I, vp, Z, vp]
    lib.attn_bwd.restype = I
    lib.attn_fwd_ex.argtypes = [vp] * 7 + [I] * 6 + [F, I, I, I, vp]
    lib.attn_fwd_ex.restype = I
    lib.attn_bwd_ex.argtypes = [vp] * 11 + [I] * 6 + [F, I, I, I, I, vp, Z, vp]
    lib.attn_bwd_ex.restype = I
    lib.attn_bwd_ex_noalloc.argtypes = [vp] * 11 + [I] * 6 + [F, I, I, I, I, vp]
    lib.attn_bwd_ex_noalloc.restype = I
    lib.attn_out_proj_bwd.argtypes = [vp] * 5 + [I] * 4 + [vp]
    lib.attn_out_proj_bwd.restype = I
    lib.attn_in_proj_bwd.argtypes = [vp] * 11 + [I] * 5 + [vp]
    lib.attn_in_proj_bwd.restype = I
    lib.attn_status_str.argtypes = [I]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = I
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().attn_status_str(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16, float16 or float32")
    return code


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, seq, dim]")


def _expect(t, name, shape, dtype):
    """The library sizes every buffer from q's dtype and (B, H, n, m, d, dv):
    a tensor of another shape or dtype would be read or written out of
    bounds, so it is refused here, before anything reaches the C ABI."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(ref, *ts):
    for t in ts:
        if t.device != ref.device:
            raise ValueError(f"all tensors must be on {ref.device}, got one on {t.device}")


def _rows_shape(B, H, rows, width, layout):
    return (B, rows, H, width) if layout == "bshd" else (B, H, rows, width)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(q, k, v, layout="bhsd"):
    """(B, H, n, m, d, dv) of [B, H, seq, dim] ("bhsd") or [B, seq, H, dim]
    ("bshd") tensors."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-d")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}, got {layout!r}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"q, k, v must share a dtype, got {q.dtype}, {k.dtype}, {v.dtype}")
    if layout == "bshd":
        q, k, v = (t.transpose(1, 2) for t in (q, k, v))   # shape arithmetic only
    B, H, n, d = q.shape
    m, dv = v.shape[2], v.shape[3]
    if tuple(k.shape) != (B, H, m, d) or tuple(v.shape[:2]) != (B, H):
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, H, n, m, d, dv


def _lens(t, B):
    """A per-batch length tensor (int32 [B] on the GPU) or None."""
    if t is None:
        return None
    if t.dtype != torch.int32 or tuple(t.shape) != (B,):
        raise ValueError(f"sequence lengths must be int32 of shape ({B},)")
    _check_dev(t)
    return t


def _mask_code(causal, mask):
    if mask is None:
        return ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE
    if causal:
        raise ValueError("give either causal=True or mask=..., not both")
    return MASKS[mask]


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, mask=None, seqlens_q=None,
        seqlens_k=None, layout="bhsd"):
    """O [B,H,n,dv] (q's dtype) and LSE [B,H,n] (float32, natural log).

    ``causal=True`` is the causal mask with n == m.  ``mask`` ("none",
    "causal" or "causal_bottom_right") and the per-batch lengths
    ``seqlens_q`` / ``seqlens_k`` (int32 [B] on the GPU) select the general
    entry point, attn_fwd_ex, and so does ``layout="bshd"`` ([B, seq, H, dim]
    tensors; LSE stays [B, H, n]).
    """
    lib = load()
    B, H, n, m, d, dv = _shape(q, k, v, layout)
    code = _dtype_code(q)
    oshape = _rows_shape(B, H, n, dv, layout)
    if out is not None:
        _expect(out, "out", oshape, q.dtype)
    if lse is not None:
        _expect(lse, "lse", (B, H, n), torch.float32)
    _check_dev(q, k, v)
    _same_device(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(oshape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    _check_dev(out, lse)
    _same_device(q, out, lse)
    if mask is None and seqlens_q is None and seqlens_k is None and layout == "bhsd":
        st = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, n, m, d, dv,
                          float(scale), int(bool(causal)), code, _stream(q))
        where = "attn_fwd"
    else:
        mcode = _mask_code(causal, mask)
        sq, sk = _lens(seqlens_q, B), _lens(seqlens_k, B)
        _same_device(q, *(t for t in (sq, sk) if t is not None))
        st = lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(sq), _ptr(sk),
                             B, H, n, m, d, dv, float(scale), mcode, LAYOUTS[layout],
                             code, _stream(q))
        where = "attn_fwd_ex"
    if st != ATTN_OK:
        raise AttnError(st, where)
    return out, lse


def _dq_flags(dq_mode, dq_split):
    if dq_mode not in DQ_MODES:
        raise ValueError(f"dq_mode must be one of {sorted(DQ_MODES)}, got {dq_mode!r}")
    flags = DQ_MODES[dq_mode]
    if dq_split is not None:
        if dq_mode != "atomic":
            raise ValueError("dq_split applies to dq_mode='atomic' only")
        if not 0 <= int(dq_split) <= DQ_SPLIT_MAX:
            raise ValueError(f"dq_split must be in 0..{DQ_SPLIT_MAX}")
        flags |= int(dq_split) << DQ_SPLIT_SHIFT
    return flags


def bwd_workspace_bytes(B, H, n, m, d, dv, dtype=torch.bfloat16, dq_mode="auto", causal=False,
                        mask=None):
    """attn_bwd_workspace_bytes_ex: workspace bytes of a backward with these
    sizes, mask (as in fwd()) and dQ mode."""
    code = _DTYPE_CODES.get(dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}; use bfloat16, float16 or float32")
    return int(load().attn_bwd_workspace_bytes_ex(B, H, n, m, d, dv, _mask_code(causal, mask),
                                                  code, _dq_flags(dq_mode, None)))


def _bwd_args(q, k, v, o, do, lse, dq, dk, dv, layout, dq_mode, dq_split, stages, scale):
    """Checks shared by bwd and bwd_noalloc; returns the sizes, dtype code,
    flags and scale."""
    B, H, n, m, d, dvw = _shape(q, k, v, layout)
    code = _dtype_code(q)
    _expect(o, "o", _rows_shape(B, H, n, dvw, layout), q.dtype)
    _expect(do, "do", _rows_shape(B, H, n, dvw, layout), q.dtype)
    _expect(lse, "lse", (B, H, n), torch.float32)
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        if t is not None:
            _expect(t, name, ref.shape, q.dtype)
    flags = _dq_flags(dq_mode, dq_split)
    _check_dev(q, k, v, o, do, lse)
    _same_device(q, k, v, o, do, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stages:
        for s_ in stages:
            flags |= STAGES[s_]
    return (B, H, n, m, d, dvw), code, flags, scale


def _outputs(q, k, v, dq, dk, dv):
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_dev(dq, dk, dv)
    _same_device(q, dq, dk, dv)
    return dq, dk, dv


def bwd(q, k, v, o, do, lse, scale=None, causal=False, dq_mode="auto", workspace=None,
        dq=None, dk=None, dv=None, stages=None, mask=None, seqlens_q=None, seqlens_k=None,
        layout="bhsd", dq_split=None):
    """(dq, dk, dv) with the shapes and dtype of (q, k, v).

    ``dq_mode`` is "auto", "separate", "atomic" or "stored_ds" (ATTN_DQ_*), and
    ``dq_split`` the number of leading 256-key blocks whose dQ the separate
    pass sums in the atomic mode.  ``stages`` (a subset of {"preprocess",
    "dkdv", "dq"}) restricts which kernels run; it exists for timing single
    kernels.  ``mask`` and the per-batch lengths and ``layout`` select
    attn_bwd_ex, as in fwd().
    """
    lib = load()
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError(f"workspace must be torch.uint8, got {workspace.dtype}")
    (B, H, n, m, d, dvw), code, flags, scale = _bwd_args(
        q, k, v, o, do, lse, dq, dk, dv, layout, dq_mode, dq_split, stages, scale)
    need = int(lib.attn_bwd_workspace_bytes_ex(B, H, n, m, d, dvw, _mask_code(causal, mask),
                                               code, flags))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_dev(workspace)
    _same_device(q, workspace)
    dq, dk, dv = _outputs(q, k, v, dq, dk, dv)
    ws_bytes = workspace.numel() * workspace.element_size()
    if mask is None and seqlens_q is None and seqlens_k is None and layout == "bhsd":
        st = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, n, m, d, dvw, float(scale),
                          int(bool(causal)), code, flags, _ptr(workspace), ws_bytes, _stream(q))
        where = "attn_bwd"
    else:
        mcode = _mask_code(causal, mask)
        sq, sk = _lens(seqlens_q, B), _lens(seqlens_k, B)
        _same_device(q, *(t for t in (sq, sk) if t is not None))
        st = lib.attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(sq), _ptr(sk), B, H, n, m, d, dvw,
                             float(scale), mcode, LAYOUTS[layout], code, flags, _ptr(workspace),
                             ws_bytes, _stream(q))
        where = "attn_bwd_ex"
    if st != ATTN_OK:
        raise AttnError(st, where)
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, dq_mode="auto",
                stages=None, mask=None, seqlens_q=None, seqlens_k=None, layout="bhsd",
                dq_split=None):
    """attn_bwd_ex_noalloc: the backward into the caller's dq, dk, dv with
    the library's static per-GPU scratch instead of a workspace (no device
    memory is allocated, here or in the library).  Calls that overlap on one
    GPU share that scratch and race.  Arguments as in bwd()."""
    lib = load()
    if dq is None or dk is None or dv is None:
        raise ValueError("bwd_noalloc writes into the caller's dq, dk and dv")
    (B, H, n, m, d, dvw), code, flags, scale = _bwd_args(
        q, k, v, o, do, lse, dq, dk, dv, layout, dq_mode, dq_split, stages, scale)
    dq, dk, dv = _outputs(q, k, v, dq, dk, dv)
    mcode = _mask_code(causal, mask)
    sq, sk = _lens(seqlens_q, B), _lens(seqlens_k, B)
    _same_device(q, *(t for t in (sq, sk) if t is not None))
    st = lib.attn_bwd_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(sq), _ptr(sk), B, H, n, m,
                                 d, dvw, float(scale), mcode, LAYOUTS[layout], code, flags,
                                 _stream(q))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_ex_noalloc")
    return dq, dk, dv


def _mat(t, rows, cols, name, dtype=None):
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must be [{rows}, {cols}], got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def out_proj_bwd(o_cat, g, w_o, dw_o=None, do_cat=None):
    """(dW_O, dO_cat) for Y = O_cat W_O and G = dL/dY: dW_O = O_cat^T G
    (float32 [H dv, d_model]) and dO_cat = G W_O^T (dtype, [T, H dv]).
    o_cat [T, H dv], g [T, d_model], w_o [H dv, d_model]; a [B, n, H, dv]
    attention output viewed as [T, H dv] is o_cat."""
    lib = load()
    T, hdv = o_cat.shape
    dm = g.shape[1]
    _mat(o_cat, T, hdv, "o_cat")
    _mat(g, T, dm, "g")
    _mat(w_o, hdv, dm, "w_o")
    if g.dtype != o_cat.dtype or w_o.dtype != o_cat.dtype:
        raise TypeError("o_cat, g and w_o must share a dtype")
    dw_o = torch.empty((hdv, dm), dtype=torch.float32, device=g.device) if dw_o is None else dw_o
    do_cat = torch.empty((T, hdv), dtype=g.dtype, device=g.device) if do_cat is None else do_cat
    _mat(dw_o, hdv, dm, "dw_o", torch.float32)
    _mat(do_cat, T, hdv, "do_cat", g.dtype)
    _check_dev(o_cat, g, w_o, dw_o, do_cat)
    _same_device(g, o_cat, w_o, dw_o, do_cat)
    st = lib.attn_out_proj_bwd(_ptr(o_cat), _ptr(g), _ptr(w_o), _ptr(dw_o), _ptr(do_cat), T, dm,
                               hdv, _dtype_code(g), _stream(g))
    if st != ATTN_OK:
        raise AttnError(st, "attn_out_proj_bwd")
    return dw_o, do_cat


def in_proj_bwd(x, w_q, w_k, w_v, dq_cat, dk_cat, dv_cat, out=None):
    """dW_Q, dW_K, dW_V (float32) and dX (dtype) for Q = X W_Q, K = X W_K,
    V = X W_V: a dict with keys dw_q, dw_k, dw_v, dx.  x [T, d_model],
    w_q, w_k [d_model, H d], w_v [d_model, H dv]; dq_cat, dk_cat [T, H d],
    dv_cat [T, H dv] (attention gradients in [B, n, H, dim] viewed as 2-d)."""
    lib = load()
    T, dm = x.shape
    hd, hdv = w_q.shape[1], w_v.shape[1]
    for t, r, c, name in ((x, T, dm, "x"), (w_q, dm, hd, "w_q"), (w_k, dm, hd, "w_k"),
                          (w_v, dm, hdv, "w_v"), (dq_cat, T, hd, "dq_cat"),
                          (dk_cat, T, hd, "dk_cat"), (dv_cat, T, hdv, "dv_cat")):
        _mat(t, r, c, name)
        if t.dtype != x.dtype:
            raise TypeError("all inputs must share a dtype")
    dev = x.device
    o = dict(out or {})
    o.setdefault("dw_q", torch.empty((dm, hd), dtype=torch.float32, device=dev))
    o.setdefault("dw_k", torch.empty((dm, hd), dtype=torch.float32, device=dev))
    o.setdefault("dw_v", torch.empty((dm, hdv), dtype=torch.float32, device=dev))
    o.setdefault("dx", torch.empty((T, dm), dtype=x.dtype, device=dev))
    for name, r, c, dt in (("dw_q", dm, hd, torch.float32), ("dw_k", dm, hd, torch.float32),
                           ("dw_v", dm, hdv, torch.float32), ("dx", T, dm, x.dtype)):
        _mat(o[name], r, c, name, dt)
    _check_dev(x, w_q, w_k, w_v, dq_cat, dk_cat, dv_cat,
               *(o[n_] for n_ in ("dw_q", "dw_k", "dw_v", "dx")))
    _same_device(x, w_q, w_k, w_v, dq_cat, dk_cat, dv_cat, *(o[n_] for n_ in ("dw_q", "dw_k", "dw_v", "dx")))
    st = lib.attn_in_proj_bwd(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(dq_cat),
                              _ptr(dk_cat), _ptr(dv_cat), _ptr(o["dw_q"]), _ptr(o["dw_k"]),
                              _ptr(o["dw_v"]), _ptr(o["dx"]), T, dm, hd, hdv, _dtype_code(x),
                              _stream(x))
    if st != ATTN_OK:
        raise AttnError(st, "attn_in_proj_bwd")
    return o

"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (no compute call runs here)."""
import ctypes
import os
import re

import pytest

import transformer_attn_bwd_amd as attn
from transformer_attn_bwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libattn.so not built")
    return attn.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(B.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.attn_version() >= 100
    for code in range(6):
        assert attn.status_str(code)
    assert "unknown" in attn.status_str(99)


def test_workspace_size(lib):
    # separate dQ pass (also what the automatic mode runs): two float32
    # arrays of B*H*round_up(n, 128) rows (rounded to 256 bytes); the atomic
    # mode adds the float32 dQ accumulator, rows x (64 or 128, the tile
    # width for d); the stored-dS mode adds 256 x 256 16-bit dS tiles:
    # N(N+1)/2 per head under a causal mask, N*M without one (N, M query and
    # key blocks of 256)
    sep, atom, sds = B.ATTN_DQ_SEPARATE, B.ATTN_DQ_ATOMIC, B.ATTN_DQ_STORED_DS
    tile = 256 * 256 * 2
    rows4k = 2 * 64 * 4096 * 4
    assert attn.bwd_workspace_bytes(2, 32, 4096, 4096, 128, 128, dq_mode="separate") == rows4k
    assert attn.bwd_workspace_bytes(2, 32, 4096, 4096, 128, 128) == rows4k
    assert attn.bwd_workspace_bytes(2, 32, 4096, 4096, 128, 128, causal=True) == rows4k
    assert attn.bwd_workspace_bytes(2, 32, 4096, 4096, 128, 128, dq_mode="atomic") == \
        64 * 4096 * 4 * (2 + 128)
    assert attn.bwd_workspace_bytes(2, 32, 4096, 4096, 128, 128, dq_mode="stored_ds") == \
        rows4k + 64 * 16 * 16 * tile
    assert attn.bwd_workspace_bytes(2, 32, 4096, 4096, 128, 128, dq_mode="stored_ds",
                                    causal=True) == rows4k + 64 * 136 * tile
    assert attn.bwd_workspace_bytes(1, 32, 16384, 16384, 128, 128, dq_mode="stored_ds",
                                    causal=True) == 2 * 32 * 16384 * 4 + 32 * 2080 * tile
    assert attn.bwd_workspace_bytes(1, 1, 1, 1, 64, 64, dq_mode="separate") == 2 * 128 * 4
    assert attn.bwd_workspace_bytes(1, 1, 1, 1, 64, 64) == 2 * 128 * 4
    assert attn.bwd_workspace_bytes(1, 1, 1, 1, 64, 64, dq_mode="stored_ds") == 2 * 128 * 4 + tile
    assert attn.bwd_workspace_bytes(1, 1, 0, 5, 64, 64) == 0
    assert attn.bwd_workspace_bytes(0, 4, 100, 5, 64, 64) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, 8, 8, 100, 100, B.ATTN_BF16, 0) == 0  # unsupported
    for code in (B.ATTN_BF16, B.ATTN_F16, B.ATTN_F32):
        assert lib.attn_bwd_workspace_bytes(2, 3, 300, 300, 64, 64, code, sep) == 2 * 6 * 384 * 4
        assert lib.attn_bwd_workspace_bytes(2, 3, 300, 300, 64, 64, code, 0) == 2 * 6 * 384 * 4
    for code in (B.ATTN_BF16, B.ATTN_F16):
        assert lib.attn_bwd_workspace_bytes(2, 3, 300, 300, 64, 64, code, atom) == \
            6 * 384 * 4 * (2 + 64)
        assert lib.attn_bwd_workspace_bytes(2, 3, 300, 300, 96, 64, code, atom) == \
            6 * 384 * 4 * (2 + 128)
        # 300 queries, 700 keys: 2 query blocks, 3 key blocks
        assert lib.attn_bwd_workspace_bytes_ex(2, 3, 300, 700, 64, 64, B.ATTN_MASK_NONE, code,
                                               sds) == 2 * 6 * 384 * 4 + 6 * 6 * tile
        assert lib.attn_bwd_workspace_bytes_ex(2, 3, 300, 700, 64, 64, B.ATTN_MASK_CAUSAL, code,
                                               sds) == 2 * 6 * 384 * 4 + 6 * 3 * tile
        assert lib.attn_bwd_workspace_bytes_ex(2, 3, 300, 300, 64, 64,
                                               B.ATTN_MASK_CAUSAL_BOTTOM_RIGHT, code, sds) == \
            2 * 6 * 384 * 4 + 6 * 3 * tile
    assert lib.attn_bwd_workspace_bytes_ex(1, 1, 8, 8, 64, 64, 3, B.ATTN_BF16, 0) == 0  # bad mask
    # the maskless size covers every mask: with more query than key blocks
    # (1024 queries, 256 keys) the causal triangle indexes more tiles (10)
    # than the dense layout (4)
    for mask, tiles in ((B.ATTN_MASK_NONE, 4), (B.ATTN_MASK_CAUSAL, 10)):
        assert lib.attn_bwd_workspace_bytes_ex(1, 1, 1024, 256, 64, 64, mask, B.ATTN_BF16,
                                               sds) == 2 * 1024 * 4 + tiles * tile
    assert lib.attn_bwd_workspace_bytes(1, 1, 1024, 256, 64, 64, B.ATTN_BF16, sds) == \
        2 * 1024 * 4 + 10 * tile
    # float32 has no fused dQ and no stored dS: nothing beyond the rows in
    # the automatic mode
    assert lib.attn_bwd_workspace_bytes(2, 3, 300, 300, 64, 64, B.ATTN_F32, 0) == 2 * 6 * 384 * 4
    assert lib.attn_bwd_workspace_bytes(1, 1, 8, 8, 64, 136, B.ATTN_F16, 0) == 0  # unsupported
    assert lib.attn_bwd_workspace_bytes(1, 1, 8, 8, 96, 40, B.ATTN_F16, 0) > 0


NULL = None
FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first


def _fwd(lib, B_=1, H=1, n=64, m=64, d=64, dv=64, scale=0.125, causal=0,
         dtype=B.ATTN_BF16, ptrs=None):
    p = ptrs if ptrs is not None else [FAKE] * 5
    return lib.attn_fwd(*p, B_, H, n, m, d, dv, scale, causal, dtype, NULL)


def _bwd(lib, B_=1, H=1, n=64, m=64, d=64, dv=64, scale=0.125, causal=0, dtype=B.ATTN_BF16,
         flags=0, ws=FAKE, ws_bytes=1 << 30, ptrs=None):
    p = ptrs if ptrs is not None else [FAKE] * 9
    return lib.attn_bwd(*p, B_, H, n, m, d, dv, scale, causal, dtype, flags, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), B.ATTN_EINVAL),
    (dict(m=0), B.ATTN_EINVAL),
    (dict(d=0), B.ATTN_EINVAL),
    (dict(B_=-2), B.ATTN_EINVAL),
    (dict(scale=float("nan")), B.ATTN_EINVAL),
    (dict(scale=float("inf")), B.ATTN_EINVAL),
    (dict(n=64, m=65, causal=1), B.ATTN_ECAUSAL_SHAPE),
    (dict(d=100, dv=100), B.ATTN_EUNSUPPORTED),    # 16-bit widths: multiples of 8
    (dict(d=64, dv=136), B.ATTN_EUNSUPPORTED),     # ... up to 128
    (dict(d=4, dv=64), B.ATTN_EUNSUPPORTED),
    (dict(dtype=7), B.ATTN_EUNSUPPORTED),
    (dict(dtype=B.ATTN_F16, d=100, dv=96), B.ATTN_EUNSUPPORTED),
    (dict(dtype=B.ATTN_F16, d=256, dv=128), B.ATTN_EUNSUPPORTED),
    (dict(dtype=B.ATTN_F32, d=129), B.ATTN_EUNSUPPORTED),
    (dict(n=(1 << 22) + 1, m=(1 << 22) + 1), B.ATTN_EUNSUPPORTED),
])
def test_fwd_rejects(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert _bwd(lib, **kw) == code


def test_null_and_misaligned_pointers(lib):
    for i in range(5):
        p = [FAKE] * 5
        p[i] = NULL
        assert _fwd(lib, ptrs=p) == B.ATTN_EINVAL
    for i in range(9):
        p = [FAKE] * 9
        p[i] = NULL
        assert _bwd(lib, ptrs=p) == B.ATTN_EINVAL
    odd = ctypes.c_void_p((1 << 20) + 2)   # not 16-byte aligned for 16-bit rows
    assert _fwd(lib, ptrs=[odd] + [FAKE] * 4) == B.ATTN_EINVAL
    assert _fwd(lib, ptrs=[odd] + [FAKE] * 4, dtype=B.ATTN_F16) == B.ATTN_EINVAL


def test_workspace_checks(lib):
    need = lib.attn_bwd_workspace_bytes(1, 1, 64, 64, 64, 64, B.ATTN_BF16, 0)
    assert _bwd(lib, ws=NULL) == B.ATTN_EWORKSPACE
    assert _bwd(lib, ws_bytes=need - 1) == B.ATTN_EWORKSPACE
    assert _bwd(lib, ws=ctypes.c_void_p((1 << 20) + 4), ws_bytes=need) == B.ATTN_EINVAL


def test_unknown_flags(lib):
    assert _bwd(lib, flags=1 << 20) == B.ATTN_EUNSUPPORTED
    assert _bwd(lib, flags=7) == B.ATTN_EUNSUPPORTED
    assert _bwd(lib, flags=4) == B.ATTN_EUNSUPPORTED
    assert _bwd(lib, flags=B.ATTN_DQ_STORED_DS | (1 << B.DQ_SPLIT_SHIFT)) == B.ATTN_EUNSUPPORTED
    # the stored-dS mode: 16-bit types only, and no diagonal that moves
    # with per-batch lengths
    assert _bwd(lib, flags=B.ATTN_DQ_STORED_DS, dtype=B.ATTN_F32) == B.ATTN_EUNSUPPORTED
    lens = ctypes.c_void_p(1 << 20)
    assert _bwd_ex(lib, flags=B.ATTN_DQ_STORED_DS, mask=B.ATTN_MASK_CAUSAL_BOTTOM_RIGHT,
                   sq=lens, sk=lens) == B.ATTN_EUNSUPPORTED
    assert _bwd_ex(lib, flags=B.ATTN_DQ_STORED_DS, mask=B.ATTN_MASK_CAUSAL_BOTTOM_RIGHT, n=64,
                   m=128) == B.ATTN_EUNSUPPORTED
    # a split only with the atomic mode; the atomic mode only for 16-bit types
    assert _bwd(lib, flags=B.ATTN_DQ_SEPARATE | (1 << B.DQ_SPLIT_SHIFT)) == B.ATTN_EUNSUPPORTED
    assert _bwd(lib, flags=B.ATTN_DQ_AUTO | (2 << B.DQ_SPLIT_SHIFT)) == B.ATTN_EUNSUPPORTED
    assert _bwd(lib, flags=B.ATTN_DQ_ATOMIC, dtype=B.ATTN_F32) == B.ATTN_EUNSUPPORTED


def test_dq_flag_constants_match_header():
    text = open(HEADER).read()
    body = re.search(r"enum attn_bwd_flags \{(.*?)\};", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    vals = dict((k.strip(), v.strip()) for k, v in (e.split("=") for e in body.split(",") if "=" in e))
    assert int(vals["ATTN_DQ_AUTO"]) == B.ATTN_DQ_AUTO == 0
    assert int(vals["ATTN_DQ_ATOMIC"]) == B.ATTN_DQ_ATOMIC == 1
    assert int(vals["ATTN_DQ_SEPARATE"]) == B.ATTN_DQ_SEPARATE == 2
    assert int(vals["ATTN_DQ_STORED_DS"]) == B.ATTN_DQ_STORED_DS == 3
    m = re.search(r"#define ATTN_DQ_SPLIT\(k\) \(\(int\)\(k\) << (\d+)\)", text)
    assert m and int(m.group(1)) == B.DQ_SPLIT_SHIFT


def test_binding_dq_split_arguments():
    assert B._dq_flags("atomic", 3) == B.ATTN_DQ_ATOMIC | (3 << B.DQ_SPLIT_SHIFT)
    assert B._dq_flags("separate", None) == B.ATTN_DQ_SEPARATE
    with pytest.raises(ValueError):
        B._dq_flags("separate", 1)
    with pytest.raises(ValueError):
        B._dq_flags("atomic", 256)
    with pytest.raises(ValueError):
        B._dq_flags("fused", None)


def test_empty_problems_need_no_pointers(lib):
    # B*H == 0: nothing to do, nothing launched, pointers may be NULL
    assert _fwd(lib, B_=0, ptrs=[NULL] * 5) == B.ATTN_OK
    assert _bwd(lib, B_=0, ptrs=[NULL] * 9, ws=NULL, ws_bytes=0) == B.ATTN_OK
    # n == 0 forward: no query rows, nothing launched
    assert _fwd(lib, n=0, ptrs=[NULL, FAKE, FAKE, NULL, NULL]) == B.ATTN_OK


def test_binding_requires_gpu_tensors():
    import torch
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libattn.so not built")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.fwd(q, q, q)


def test_binding_dtype_codes():
    import torch
    assert B._dtype_code(torch.zeros(1, dtype=torch.float16)) == B.ATTN_F16
    assert B._dtype_code(torch.zeros(1, dtype=torch.bfloat16)) == B.ATTN_BF16
    assert B._dtype_code(torch.zeros(1, dtype=torch.float32)) == B.ATTN_F32
    with pytest.raises(TypeError):
        B._dtype_code(torch.zeros(1, dtype=torch.float64))


def test_binding_constants_match_header():
    text = open(HEADER).read()
    body = re.search(r"enum attn_dtype \{([^}]*)\}", text).group(1)
    vals = dict((k.strip(), int(v)) for k, v in (e.split("=") for e in body.split(",")))
    assert vals == {"ATTN_F32": B.ATTN_F32, "ATTN_BF16": B.ATTN_BF16, "ATTN_F16": B.ATTN_F16}


def _fwd_ex(lib, B_=1, H=1, n=64, m=64, d=64, dv=64, scale=0.125, mask=0, layout=0,
            dtype=B.ATTN_BF16, sq=None, sk=None, ptrs=None):
    p = ptrs if ptrs is not None else [FAKE] * 5
    return lib.attn_fwd_ex(*p, sq, sk, B_, H, n, m, d, dv, scale, mask, layout, dtype, NULL)


def _bwd_ex(lib, B_=1, H=1, n=64, m=64, d=64, dv=64, scale=0.125, mask=0, layout=0,
            dtype=B.ATTN_BF16, flags=0, sq=None, sk=None, ws=FAKE, ws_bytes=1 << 30, ptrs=None):
    p = ptrs if ptrs is not None else [FAKE] * 9
    return lib.attn_bwd_ex(*p, sq, sk, B_, H, n, m, d, dv, scale, mask, layout, dtype, flags,
                           ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=3), B.ATTN_EUNSUPPORTED),
    (dict(mask=-1), B.ATTN_EUNSUPPORTED),
    (dict(n=-1), B.ATTN_EINVAL),
    (dict(m=0), B.ATTN_EINVAL),
    (dict(scale=float("nan")), B.ATTN_EINVAL),
    (dict(d=100, dv=96), B.ATTN_EUNSUPPORTED),
    (dict(layout=2), B.ATTN_EUNSUPPORTED),
    (dict(layout=B.ATTN_LAYOUT_BSHD, H=4096, n=1 << 20, m=1 << 20, d=128, dv=128),
     B.ATTN_EUNSUPPORTED),   # a head's rows would span more than 2^30 bytes
    (dict(sq=ctypes.c_void_p((1 << 20) + 2)), B.ATTN_EINVAL),
    (dict(sk=ctypes.c_void_p((1 << 20) + 1)), B.ATTN_EINVAL),
])
def test_ex_rejects(lib, kw, code):
    assert _fwd_ex(lib, **kw) == code
    assert _bwd_ex(lib, **kw) == code


def test_ex_empty_problem_needs_no_pointers(lib):
    # B*H == 0 with causal n != m: valid for the _ex entry points, nothing launched
    assert _fwd_ex(lib, B_=0, n=3, m=70, mask=B.ATTN_MASK_CAUSAL_BOTTOM_RIGHT,
                   ptrs=[NULL] * 5) == B.ATTN_OK
    assert _bwd_ex(lib, B_=0, n=3, m=70, mask=B.ATTN_MASK_CAUSAL, ptrs=[NULL] * 9, ws=NULL,
                   ws_bytes=0) == B.ATTN_OK
    # the plain entry points still reject causal n != m
    assert _fwd(lib, B_=0, n=3, m=70, causal=1, ptrs=[NULL] * 5) == B.ATTN_ECAUSAL_SHAPE


def test_binding_mask_arguments():
    with pytest.raises(ValueError):
        B._mask_code(True, "causal")
    assert B._mask_code(False, None) == B.ATTN_MASK_NONE
    assert B._mask_code(True, None) == B.ATTN_MASK_CAUSAL
    assert B._mask_code(False, "causal_bottom_right") == B.ATTN_MASK_CAUSAL_BOTTOM_RIGHT
    with pytest.raises(KeyError):
        B._mask_code(False, "sliding_window")


def test_mask_constants_match_header():
    text = open(HEADER).read()
    body = re.search(r"enum attn_mask \{(.*?)\};", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    vals = dict((k.strip(), int(v)) for k, v in (e.split("=") for e in body.split(",") if "=" in e))
    assert vals == {"ATTN_MASK_NONE": B.ATTN_MASK_NONE, "ATTN_MASK_CAUSAL": B.ATTN_MASK_CAUSAL,
                    "ATTN_MASK_CAUSAL_BOTTOM_RIGHT": B.ATTN_MASK_CAUSAL_BOTTOM_RIGHT}


def test_layout_constants_match_header():
    text = open(HEADER).read()
    body = re.search(r"enum attn_layout \{(.*?)\};", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    vals = dict((k.strip(), int(v)) for k, v in (e.split("=") for e in body.split(",") if "=" in e))
    assert vals == {"ATTN_LAYOUT_BHSD": B.ATTN_LAYOUT_BHSD, "ATTN_LAYOUT_BSHD": B.ATTN_LAYOUT_BSHD}


def _outp(lib, T=64, dm=64, hdv=64, dtype=B.ATTN_BF16, ptrs=None):
    p = ptrs if ptrs is not None else [FAKE] * 5
    return lib.attn_out_proj_bwd(*p, T, dm, hdv, dtype, NULL)


def _inp(lib, T=64, dm=64, hd=64, hdv=64, dtype=B.ATTN_BF16, ptrs=None):
    p = ptrs if ptrs is not None else [FAKE] * 11
    return lib.attn_in_proj_bwd(*p, T, dm, hd, hdv, dtype, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=B.ATTN_F32), B.ATTN_EUNSUPPORTED),
    (dict(T=-1), B.ATTN_EINVAL),
    (dict(dm=0), B.ATTN_EINVAL),
    (dict(dm=60), B.ATTN_EUNSUPPORTED),          # rows must be whole 16-byte chunks
    (dict(hdv=100), B.ATTN_EUNSUPPORTED),
    (dict(T=1 << 20, dm=1024), B.ATTN_EUNSUPPORTED),   # a matrix over 2^30 bytes
])
def test_proj_rejects(lib, kw, code):
    assert _outp(lib, **kw) == code
    assert _inp(lib, **kw) == code


def test_proj_null_and_misaligned(lib):
    for i in range(5):
        p = [FAKE] * 5
        p[i] = NULL
        assert _outp(lib, ptrs=p) == B.ATTN_EINVAL
    for i in range(11):
        p = [FAKE] * 11
        p[i] = ctypes.c_void_p((1 << 20) + 8)
        assert _inp(lib, ptrs=p) == B.ATTN_EINVAL


# The binding sizes nothing itself: every tensor it passes on must have the
# shape and dtype the library derives from q.  These checks run before the
# device check, so CPU tensors exercise them here.
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def _bwd_args(**over):
    import torch
    a = dict(q=_t(1, 2, 8, 64), k=_t(1, 2, 16, 64), v=_t(1, 2, 16, 32), o=_t(1, 2, 8, 32),
             do=_t(1, 2, 8, 32), lse=_t(1, 2, 8, dtype=torch.float32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,exc", [
    (dict(k=_t(1, 2, 16, 64, dtype=None).float()), TypeError),      # k dtype != q dtype
    (dict(v=_t(1, 2, 16, 32).half()), TypeError),
    (dict(o=_t(1, 2, 8, 64)), ValueError),                            # o width != dv
    (dict(o=_t(1, 2, 8, 32).half()), TypeError),
    (dict(do=_t(1, 2, 9, 32)), ValueError),                           # do rows != n
    (dict(lse=_t(1, 2, 8)), TypeError),                               # lse must be float32
    (dict(lse=_t(1, 2, 7).float()), ValueError),
    (dict(dq=_t(1, 2, 8, 32)), ValueError),                           # dq must match q
    (dict(dk=_t(1, 2, 16, 64).float()), TypeError),
    (dict(dv=_t(1, 2, 15, 32)), ValueError),
    (dict(workspace=_t(16).float()), TypeError),
    (dict(dq_mode="bogus"), ValueError),
])
def test_binding_bwd_rejects_mismatched_tensors(over, exc):
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libattn.so not built")
    with pytest.raises(exc):
        attn.bwd(**_bwd_args(**over))


@pytest.mark.parametrize("over,exc", [
    (dict(out=_t(1, 2, 8, 64)), ValueError),
    (dict(out=_t(1, 2, 8, 32).half()), TypeError),
    (dict(lse=_t(1, 2, 8)), TypeError),
    (dict(lse=_t(2, 1, 8).float()), ValueError),
    (dict(k=_t(1, 2, 16, 64).half()), TypeError),
    (dict(layout="sbhd"), ValueError),
])
def test_binding_fwd_rejects_mismatched_tensors(over, exc):
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libattn.so not built")
    a = dict(q=_t(1, 2, 8, 64), k=_t(1, 2, 16, 64), v=_t(1, 2, 16, 32))
    a.update(over)
    with pytest.raises(exc):
        attn.fwd(**a)


def test_binding_bshd_shapes_checked():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libattn.so not built")
    q, k, v = _t(1, 8, 2, 64), _t(1, 16, 2, 64), _t(1, 16, 2, 32)
    with pytest.raises(ValueError):   # a [B, H, n, dv] o given to a [B, n, H, dim] call
        attn.bwd(q, k, v, _t(1, 2, 8, 32), _t(1, 8, 2, 32), _t(1, 2, 8).float(), layout="bshd")
    with pytest.raises(ValueError):   # shapes right, tensors on the CPU
        attn.bwd(q, k, v, _t(1, 8, 2, 32), _t(1, 8, 2, 32), _t(1, 2, 8).float(), layout="bshd")


def test_binding_proj_rejects_mismatched_outputs():
    import torch
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libattn.so not built")
    T, dm, hd = 16, 32, 32
    with pytest.raises(TypeError):    # dW_O must be float32
        attn.out_proj_bwd(_t(T, hd), _t(T, dm), _t(hd, dm), dw_o=_t(hd, dm))
    with pytest.raises(TypeError):    # dO_cat in the input dtype
        attn.out_proj_bwd(_t(T, hd), _t(T, dm), _t(hd, dm), do_cat=_t(T, hd).float())
    with pytest.raises(ValueError):
        attn.in_proj_bwd(_t(T, dm), _t(dm, hd), _t(dm, hd), _t(dm, hd), _t(T, hd), _t(T, hd),
                         _t(T, hd), out={"dx": _t(T, dm + 8)})
    with pytest.raises(TypeError):
        attn.in_proj_bwd(_t(T, dm), _t(dm, hd), _t(dm, hd), _t(dm, hd), _t(T, hd), _t(T, hd),
                         _t(T, hd), out={"dw_k": _t(dm, hd)})

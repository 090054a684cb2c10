// C ABI of libattn: argument validation, workspace carving and dispatch to
// the gfx950 kernels.  Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "attn.h"
#include "attn_launch.h"

// The no-allocation backward's scratch: one array per GPU, held for the
// life of the process.  Host code never passes `scratch` itself to a kernel
// (on the host it names a stand-in, not device memory); it passes the
// device address that scratch_addr() looks up once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

using attn::Problem;
using attn::Workspace;

constexpr int kMaxSeq = 1 << 22;          // n, m limit (grid y dimension and int math)
constexpr int kStageMask = ATTN_STAGE_PREPROCESS | ATTN_STAGE_DKDV | ATTN_STAGE_DQ;
constexpr int kDqModeMask = 0xF;
constexpr int kSplitShift = 12;
constexpr int kSplitMask = 0xFF << kSplitShift;
static_assert(ATTN_DQ_SPLIT(1) == 1 << kSplitShift, "split field of the C ABI");

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool is_16bit(int dtype) { return dtype == ATTN_BF16 || dtype == ATTN_F16; }

static_assert(ATTN_F32 == attn::kDtypeF32 && ATTN_BF16 == attn::kDtypeBF16 &&
                  ATTN_F16 == attn::kDtypeF16,
              "dtype codes of the C ABI and the kernels agree");
static_assert(ATTN_MASK_NONE == attn::kMaskNone && ATTN_MASK_CAUSAL == attn::kMaskCausal &&
                  ATTN_MASK_CAUSAL_BOTTOM_RIGHT == attn::kMaskCausalBottomRight,
              "mask codes of the C ABI and the kernels agree");

// Sizes, dtype, head widths, mask mode and scale; shared by fwd and bwd.
int check_problem(int B, int H, int n, int m, int d, int dv, float scale, int mask, int dtype,
                  Problem* out) {
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_EUNSUPPORTED;
    if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL && mask != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
        return ATTN_EUNSUPPORTED;
    if (B < 0 || H < 0 || n < 0 || m < 1 || d < 1 || dv < 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    if (n > kMaxSeq || m > kMaxSeq) return ATTN_EUNSUPPORTED;
    if (is_16bit(dtype)) {
        // head widths padded to 64 or 128 columns inside the kernels
        const bool ok = d <= 128 && dv <= 128 && d % 8 == 0 && dv % 8 == 0;
        if (!ok) return ATTN_EUNSUPPORTED;
        if ((long)B * H > 0x7fffffffL) return ATTN_EUNSUPPORTED;
    } else {
        if (d > 128 || dv > 128) return ATTN_EUNSUPPORTED;
        if ((long)B * H > 65535L) return ATTN_EUNSUPPORTED;
    }
    out->B = B;
    out->H = H;
    out->n = n;
    out->m = m;
    out->d = d;
    out->dv = dv;
    out->scale = scale;
    out->mask = mask;
    out->causal = mask != ATTN_MASK_NONE;
    out->dtype = dtype;
    return ATTN_OK;
}

// Per-batch length arrays: NULL, or 4-byte aligned device memory.
bool lens_ok(const int* p) { return p == nullptr || aligned(p, 4); }

// Memory layout of the tensors; the 16-bit kernels address one head's rows
// through 32-bit buffer offsets, so a head's byte range must stay within
// 2^30 (always true for [B, H, seq, dim]).
int set_layout(Problem* p, int layout) {
    if (layout != ATTN_LAYOUT_BHSD && layout != ATTN_LAYOUT_BSHD) return ATTN_EUNSUPPORTED;
    p->bshd = layout == ATTN_LAYOUT_BSHD;
    if (p->bshd && p->dtype != ATTN_F32) {
        const long rows = p->n > p->m ? p->n : p->m, w = p->d > p->dv ? p->d : p->dv;
        if (rows * p->H * w * 2 > (1L << 30)) return ATTN_EUNSUPPORTED;
    }
    return ATTN_OK;
}

// A tensor with elements needs a non-null pointer aligned for the kernels'
// vector accesses (16 bytes for 16-bit rows, 4 bytes for float32).
bool tensor_ok(const void* p, long elems, int dtype) {
    if (elems == 0) return true;
    if (p == nullptr) return false;
    return aligned(p, is_16bit(dtype) ? 16 : 4);
}

// Width of the float32 dQ accumulator's rows: the 16-bit kernels' tile
// width for d.
int acc_width(const Problem& p) { return (attn::mfma_widths(p) >> 8) == 0x40 ? 64 : 128; }

// Whether the stored dS tiles of a problem are indexed triangularly.
bool ds_tri(const Problem& p) { return p.causal; }

// Bytes of one head's stored dS tiles (16-bit, 256 x 256 each).
size_t ds_head_bytes(const Problem& p) {
    return (size_t)attn::ds_tiles_per_head(p.n, p.m, ds_tri(p)) * attn::kDsTile * attn::kDsTile *
           2;
}
constexpr size_t kMaxDsHeadBytes = (size_t)1 << 31;

// Stored-dS mode: dS tiles are indexed triangularly when the causal
// diagonal is j = i in every batch element (top-left, or bottom-right
// with n == m and no per-batch lengths), densely without a mask; a
// bottom-right diagonal that can move per batch element is not supported.
bool ds_supported(const Problem& p) {
    if (!is_16bit(p.dtype) || attn::mfma_widths(p) == 0) return false;
    if (p.mask == ATTN_MASK_CAUSAL_BOTTOM_RIGHT &&
        (p.n != p.m || p.seqlens_q != nullptr || p.seqlens_k != nullptr))
        return false;
    // one head's tiles are addressed with 32-bit byte offsets
    return ds_head_bytes(p) <= kMaxDsHeadBytes;
}

size_t ds_bytes(const Problem& p) {
    return round_up((size_t)p.heads() * ds_head_bytes(p), 256);
}

// The concrete dQ mode of a call: ATTN_DQ_SEPARATE, ATTN_DQ_ATOMIC or
// ATTN_DQ_STORED_DS (float32 always runs the separate pass).  ATTN_DQ_AUTO
// is the separate pass: on MI355X it measured fastest at every workload
// shape timed (causal n = 1k to 16k at d = 64 and 128, cross 512 x 2048),
// ahead of the atomic mode at its best split and of the stored-dS mode.
int resolve_mode(const Problem& p, int flags) {
    const int mode = flags & kDqModeMask;
    if (!is_16bit(p.dtype)) return ATTN_DQ_SEPARATE;
    return mode == ATTN_DQ_AUTO ? ATTN_DQ_SEPARATE : mode;
}

size_t workspace_bytes(const Problem& p, int flags) {
    if (p.heads() == 0 || p.n == 0) return 0;
    const size_t rows = (size_t)p.heads() * (size_t)attn::padded_rows(p.n);
    size_t bytes = round_up(2 * rows * sizeof(float), 256);
    const int mode = resolve_mode(p, flags);
    if (mode == ATTN_DQ_ATOMIC) bytes += round_up(rows * acc_width(p) * sizeof(float), 256);
    if (mode == ATTN_DQ_STORED_DS) bytes += ds_bytes(p);
    return bytes;
}

// How dQ is accumulated for a 16-bit backward in the atomic mode: the
// number of leading 256-key blocks the separate pass sums before the fused
// dK/dV kernel adds the rest with atomics; -1 in the other modes.
int resolve_dq(const Problem& p, int flags) {
    if (resolve_mode(p, flags) != ATTN_DQ_ATOMIC) return -1;
    return (flags & kSplitMask) >> kSplitShift;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array.
int scratch_addr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return ATTN_EUNSUPPORTED;
    void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
                (void)hipGetLastError();
                return ATTN_EHIP;
            }
            g_scratch_addr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return ATTN_OK;
}

int hip_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

constexpr int kNoKeyLimit = 0x7fffffff;

// The 16-bit backward with the fused dQ: the separate pass over the keys of
// the first `split` 256-key blocks (with the preprocess in its prologue)
// initialises the float32 accumulator, the dK/dV kernel adds dS K for the
// later key blocks with atomics, and the convert pass writes dq.
template <typename T>
int bwd_atomic_t(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv_out,
                 const attn::Workspace& w, int split, int stages, hipStream_t s) {
    const long lim = (long)split * attn::kDkdvBlock;
    const int key_limit = lim > kNoKeyLimit ? kNoKeyLimit : (int)lim;
    const bool pre = (stages & ATTN_STAGE_PREPROCESS) != 0, dqs = (stages & ATTN_STAGE_DQ) != 0;
    int st;
    if (p.n > 0 && dqs) {
        if (!attn::launch_bwd_dq_mfma<T>(p, q, k, v, dout, pre ? o : nullptr, pre ? lse : nullptr,
                                         w, nullptr, w.dqacc, key_limit, s))
            return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    } else if (p.n > 0 && pre) {
        if (!attn::launch_bwd_preprocess_mfma<T>(p, o, dout, lse, w, s)) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (stages & ATTN_STAGE_DKDV) {
        if (!attn::launch_bwd_dkdv_dqa_mfma<T>(p, q, k, v, dout, w, dk, dv_out, w.dqacc, key_limit,
                                               s))
            return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (p.n > 0 && dqs) {
        attn::launch_dq_convert<T>(p, w, dq, s);
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    return ATTN_OK;
}

int bwd_atomic(const Problem& p, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv_out,
               const attn::Workspace& w, int split, int stages, hipStream_t s) {
    return p.dtype == ATTN_BF16
               ? bwd_atomic_t<__bf16>(p, q, k, v, o, dout, lse, dq, dk, dv_out, w, split, stages, s)
               : bwd_atomic_t<_Float16>(p, q, k, v, o, dout, lse, dq, dk, dv_out, w, split, stages,
                                        s);
}

// The 16-bit backward in the stored-dS mode: the preprocess, the dK/dV
// kernel that also writes dS to the workspace's tiles, and dQ = scale dS K
// from those tiles.
template <typename T>
int bwd_stored_t(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv_out,
                 const attn::Workspace& w, int stages, hipStream_t s) {
    int st;
    if (p.n > 0 && (stages & ATTN_STAGE_PREPROCESS)) {
        if (!attn::launch_bwd_preprocess_mfma<T>(p, o, dout, lse, w, s)) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (stages & ATTN_STAGE_DKDV) {
        if (!attn::launch_bwd_dkdv_dss_mfma<T>(p, q, k, v, dout, w, dk, dv_out, s))
            return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (p.n > 0 && (stages & ATTN_STAGE_DQ)) {
        if (!attn::launch_bwd_dq_ds_mfma<T>(p, k, w, dq, s)) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    return ATTN_OK;
}

int bwd_stored(const Problem& p, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv_out,
               const attn::Workspace& w, int stages, hipStream_t s) {
    return p.dtype == ATTN_BF16
               ? bwd_stored_t<__bf16>(p, q, k, v, o, dout, lse, dq, dk, dv_out, w, stages, s)
               : bwd_stored_t<_Float16>(p, q, k, v, o, dout, lse, dq, dk, dv_out, w, stages, s);
}

// Sizes of the projection calls: T >= 0, widths multiples of 8 (16-byte
// rows), every matrix within 2^30 bytes (32-bit buffer offsets).
int check_proj(int T, int d_model, int hd, int hdv, int dtype, attn::ProjProblem* p) {
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_EUNSUPPORTED;
    if (T < 0 || d_model < 8 || hd < 8 || hdv < 8) return ATTN_EINVAL;
    if (d_model % 8 || hd % 8 || hdv % 8) return ATTN_EUNSUPPORTED;
    const long widest = d_model > hd ? (d_model > hdv ? d_model : hdv) : (hd > hdv ? hd : hdv);
    const long rows = T > d_model ? T : d_model;
    if (rows * widest * 2 > (1L << 30) || (long)hd * d_model * 4 > (1L << 30) ||
        (long)hdv * d_model * 4 > (1L << 30))
        return ATTN_EUNSUPPORTED;
    p->T = T;
    p->d_model = d_model;
    p->hd = hd;
    p->hdv = hdv;
    return ATTN_OK;
}

bool mat_ok(const void* p, long elems, size_t align) {
    if (elems == 0) return true;
    return p != nullptr && aligned(p, align);
}

}  // namespace

extern "C" {

int attn_version(void) { return 100; }

const char* attn_status_str(int status) {
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument (null or misaligned pointer, bad size or scale)";
    case ATTN_ECAUSAL_SHAPE: return "causal masking requires n == m";
    case ATTN_EUNSUPPORTED: return "unsupported dtype, head widths, size or flags";
    case ATTN_EWORKSPACE: return "workspace missing or too small";
    case ATTN_EHIP: return "HIP launch failed";
    case ATTN_ESCRATCH: return "problem needs more scratch than the no-allocation call's static array";
    default: return "unknown status";
    }
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                const int* seqlens_q, const int* seqlens_k, int B, int H, int n, int m, int d,
                int dv, float scale, int mask, int layout, int dtype, void* stream) {
    Problem p;
    int st = check_problem(B, H, n, m, d, dv, scale, mask, dtype, &p);
    if (st != ATTN_OK) return st;
    if ((st = set_layout(&p, layout)) != ATTN_OK) return st;
    if (!lens_ok(seqlens_q) || !lens_ok(seqlens_k)) return ATTN_EINVAL;
    p.seqlens_q = seqlens_q;
    p.seqlens_k = seqlens_k;
    const long hq = p.heads() * (long)n, hk = p.heads() * (long)m;
    if (!tensor_ok(q, hq * d, dtype) || !tensor_ok(k, hk * d, dtype) ||
        !tensor_ok(v, hk * dv, dtype) || !tensor_ok(o, hq * dv, dtype) ||
        !tensor_ok(lse, hq, ATTN_F32))
        return ATTN_EINVAL;
    if (hq == 0) return ATTN_OK;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    bool ok = is_16bit(dtype)
                  ? (dtype == ATTN_BF16 ? attn::launch_fwd_mfma<__bf16>(p, q, k, v, o, lse, s)
                                        : attn::launch_fwd_mfma<_Float16>(p, q, k, v, o, lse, s))
                  : attn::launch_fwd_f32(p, (const float*)q, (const float*)k, (const float*)v,
                                         (float*)o, lse, s);
    if (!ok) return ATTN_EUNSUPPORTED;
    return hip_status();
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int n, int m, int d, int dv, float scale, int causal, int dtype, void* stream) {
    Problem p;
    int st = check_problem(B, H, n, m, d, dv, scale, causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE,
                           dtype, &p);
    if (st != ATTN_OK) return st;
    if (causal && n != m) return ATTN_ECAUSAL_SHAPE;
    return attn_fwd_ex(q, k, v, o, lse, nullptr, nullptr, B, H, n, m, d, dv, scale,
                       causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE, ATTN_LAYOUT_BHSD, dtype,
                       stream);
}

size_t attn_bwd_workspace_bytes_ex(int B, int H, int n, int m, int d, int dv, int mask,
                                   int dtype, int flags) {
    Problem p;
    if (check_problem(B, H, n, m, d, dv, 1.f, mask, dtype, &p) != ATTN_OK) return 0;
    return workspace_bytes(p, flags);
}

size_t attn_bwd_workspace_bytes(int B, int H, int n, int m, int d, int dv, int dtype,
                                int flags) {
    // without the mask: enough for every mask mode (the dense stored-dS
    // layout is the larger one unless there are more query than key blocks)
    const size_t dense =
        attn_bwd_workspace_bytes_ex(B, H, n, m, d, dv, ATTN_MASK_NONE, dtype, flags);
    const size_t tri =
        attn_bwd_workspace_bytes_ex(B, H, n, m, d, dv, ATTN_MASK_CAUSAL, dtype, flags);
    return dense > tri ? dense : tri;
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv_out, const int* seqlens_q,
                const int* seqlens_k, int B, int H, int n, int m, int d, int dv, float scale,
                int mask, int layout, int dtype, int flags, void* workspace,
                size_t workspace_bytes_given, void* stream) {
    Problem p;
    int st = check_problem(B, H, n, m, d, dv, scale, mask, dtype, &p);
    if (st != ATTN_OK) return st;
    if ((st = set_layout(&p, layout)) != ATTN_OK) return st;
    if (!lens_ok(seqlens_q) || !lens_ok(seqlens_k)) return ATTN_EINVAL;
    p.seqlens_q = seqlens_q;
    p.seqlens_k = seqlens_k;
    if (flags & ~(kDqModeMask | kStageMask | kSplitMask)) return ATTN_EUNSUPPORTED;
    const int dq_mode = flags & kDqModeMask;
    if (dq_mode != ATTN_DQ_AUTO && dq_mode != ATTN_DQ_SEPARATE && dq_mode != ATTN_DQ_ATOMIC &&
        dq_mode != ATTN_DQ_STORED_DS)
        return ATTN_EUNSUPPORTED;
    if ((flags & kSplitMask) && dq_mode != ATTN_DQ_ATOMIC) return ATTN_EUNSUPPORTED;
    if (dq_mode == ATTN_DQ_ATOMIC && !is_16bit(dtype)) return ATTN_EUNSUPPORTED;
    if (dq_mode == ATTN_DQ_STORED_DS && !ds_supported(p)) return ATTN_EUNSUPPORTED;
    const long hq = p.heads() * (long)n, hk = p.heads() * (long)m;
    if (!tensor_ok(q, hq * d, dtype) || !tensor_ok(k, hk * d, dtype) ||
        !tensor_ok(v, hk * dv, dtype) || !tensor_ok(o, hq * dv, dtype) ||
        !tensor_ok(dout, hq * dv, dtype) || !tensor_ok(lse, hq, ATTN_F32) ||
        !tensor_ok(dq, hq * d, dtype) || !tensor_ok(dk, hk * d, dtype) ||
        !tensor_ok(dv_out, hk * dv, dtype))
        return ATTN_EINVAL;
    const size_t need = workspace_bytes(p, flags);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes_given < need) return ATTN_EWORKSPACE;
        if (!aligned(workspace, 16)) return ATTN_EINVAL;
    }
    if (p.heads() == 0) return ATTN_OK;

    int stages = flags & kStageMask;
    if (stages == 0) stages = kStageMask;
    Workspace w;
    w.n_pad = attn::padded_rows(n);
    w.lse2 = (float*)workspace;
    w.D = w.lse2 + (size_t)p.heads() * (size_t)w.n_pad;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();

    const bool bf = is_16bit(dtype);
    if (resolve_mode(p, flags) == ATTN_DQ_STORED_DS) {
        const size_t head = ds_head_bytes(p);
        w.ds.p = (char*)workspace + round_up(2 * (size_t)p.heads() * w.n_pad * 4, 256);
        w.ds.head_elems = (long)(head / 2);
        w.ds.tri = ds_tri(p) ? 1 : 0;
        w.ds.mblk = (m + attn::kDsTile - 1) / attn::kDsTile;
        return bwd_stored(p, q, k, v, o, dout, lse, dq, dk, dv_out, w, stages, s);
    }
    const int split = resolve_dq(p, flags);
    if (split >= 0) {
        w.dqacc = (float*)((char*)workspace + round_up(2 * (size_t)p.heads() * w.n_pad * 4, 256));
        w.acc_w = acc_width(p);
        return bwd_atomic(p, q, k, v, o, dout, lse, dq, dk, dv_out, w, split, stages, s);
    }
    // 16-bit calls that run both the preprocess and the dQ pass fold the
    // former into the latter's prologue (same bits), which then runs before
    // the dK/dV kernel that reads its results.
    const bool fused =
        bf && n > 0 && (stages & ATTN_STAGE_PREPROCESS) && (stages & ATTN_STAGE_DQ);
    bool ok = true;
    if (fused) {
        ok = dtype == ATTN_BF16
                 ? attn::launch_bwd_dq_mfma<__bf16>(p, q, k, v, dout, o, lse, w, dq, nullptr,
                                                    kNoKeyLimit, s)
                 : attn::launch_bwd_dq_mfma<_Float16>(p, q, k, v, dout, o, lse, w, dq, nullptr,
                                                      kNoKeyLimit, s);
        if (!ok) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (n > 0 && (stages & ATTN_STAGE_PREPROCESS) && !fused) {
        ok = bf ? (dtype == ATTN_BF16
                       ? attn::launch_bwd_preprocess_mfma<__bf16>(p, o, dout, lse, w, s)
                       : attn::launch_bwd_preprocess_mfma<_Float16>(p, o, dout, lse, w, s))
                : attn::launch_bwd_preprocess_f32(p, (const float*)o, (const float*)dout, lse, w, s);
        if (!ok) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (stages & ATTN_STAGE_DKDV) {
        // With n == 0 the kernel visits no query tile and writes zeros.
        ok = bf ? (dtype == ATTN_BF16
                       ? attn::launch_bwd_dkdv_mfma<__bf16>(p, q, k, v, dout, w, dk, dv_out, s)
                       : attn::launch_bwd_dkdv_mfma<_Float16>(p, q, k, v, dout, w, dk, dv_out, s))
                : attn::launch_bwd_dkdv_f32(p, (const float*)q, (const float*)k, (const float*)v,
                                            (const float*)dout, w, (float*)dk, (float*)dv_out, s);
        if (!ok) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    if (n > 0 && (stages & ATTN_STAGE_DQ) && !fused) {
        ok = bf ? (dtype == ATTN_BF16
                       ? attn::launch_bwd_dq_mfma<__bf16>(p, q, k, v, dout, nullptr, nullptr,
                                                          w, dq, nullptr, kNoKeyLimit, s)
                       : attn::launch_bwd_dq_mfma<_Float16>(p, q, k, v, dout, nullptr, nullptr,
                                                            w, dq, nullptr, kNoKeyLimit, s))
                : attn::launch_bwd_dq_f32(p, (const float*)q, (const float*)k, (const float*)v,
                                          (const float*)dout, w, (float*)dq, s);
        if (!ok) return ATTN_EUNSUPPORTED;
        if ((st = hip_status()) != ATTN_OK) return st;
    }
    return ATTN_OK;
}

int attn_bwd_ex_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv_out,
                        const int* seqlens_q, const int* seqlens_k, int B, int H, int n, int m,
                        int d, int dv, float scale, int mask, int layout, int dtype, int flags,
                        void* stream) {
    Problem p;
    int st = check_problem(B, H, n, m, d, dv, scale, mask, dtype, &p);
    if (st != ATTN_OK) return st;
    if (flags & ~(kDqModeMask | kStageMask | kSplitMask)) return ATTN_EUNSUPPORTED;
    p.seqlens_q = seqlens_q;
    p.seqlens_k = seqlens_k;
    // ATTN_DQ_AUTO becomes the mode it resolves to (the separate pass), so
    // that the size check below is that of the mode that runs.
    if ((flags & kDqModeMask) == ATTN_DQ_AUTO) {
        flags &= ~(kDqModeMask | kSplitMask);
        flags |= ATTN_DQ_SEPARATE;
    }
    const size_t need = workspace_bytes(p, flags);
    if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ESCRATCH;
    void* ws = nullptr;
    if (need > 0 && (st = scratch_addr(&ws)) != ATTN_OK) return st;
    return attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv_out, seqlens_q, seqlens_k, B, H, n, m,
                       d, dv, scale, mask, layout, dtype, flags, ws, ATTN_NOALLOC_SCRATCH_BYTES,
                       stream);
}

int attn_out_proj_bwd(const void* o_cat, const void* g, const void* w_o, float* dw_o,
                      void* do_cat, int T, int d_model, int hdv, int dtype, void* stream) {
    attn::ProjProblem p;
    int st = check_proj(T, d_model, 8, hdv, dtype, &p);
    if (st != ATTN_OK) return st;
    const long t = T;
    if (!mat_ok(o_cat, t * hdv, 16) || !mat_ok(g, t * d_model, 16) ||
        !mat_ok(w_o, (long)hdv * d_model, 16) || !mat_ok(dw_o, (long)hdv * d_model, 16) ||
        !mat_ok(do_cat, t * hdv, 16))
        return ATTN_EINVAL;
    (void)hipGetLastError();
    if (dtype == ATTN_BF16)
        attn::launch_out_proj_bwd<__bf16>(p, o_cat, g, w_o, dw_o, do_cat, (hipStream_t)stream);
    else
        attn::launch_out_proj_bwd<_Float16>(p, o_cat, g, w_o, dw_o, do_cat, (hipStream_t)stream);
    return hip_status();
}

int attn_in_proj_bwd(const void* x, const void* w_q, const void* w_k, const void* w_v,
                     const void* dq_cat, const void* dk_cat, const void* dv_cat, float* dw_q,
                     float* dw_k, float* dw_v, void* dx, int T, int d_model, int hd, int hdv,
                     int dtype, void* stream) {
    attn::ProjProblem p;
    int st = check_proj(T, d_model, hd, hdv, dtype, &p);
    if (st != ATTN_OK) return st;
    const long t = T, dm = d_model;
    if (!mat_ok(x, t * dm, 16) || !mat_ok(w_q, dm * hd, 16) || !mat_ok(w_k, dm * hd, 16) ||
        !mat_ok(w_v, dm * hdv, 16) || !mat_ok(dq_cat, t * hd, 16) ||
        !mat_ok(dk_cat, t * hd, 16) || !mat_ok(dv_cat, t * hdv, 16) ||
        !mat_ok(dw_q, dm * hd, 16) || !mat_ok(dw_k, dm * hd, 16) ||
        !mat_ok(dw_v, dm * hdv, 16) || !mat_ok(dx, t * dm, 16))
        return ATTN_EINVAL;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    if (dtype == ATTN_BF16)
        attn::launch_in_proj_bwd<__bf16>(p, x, w_q, w_k, w_v, dq_cat, dk_cat, dv_cat, dw_q, dw_k,
                                         dw_v, dx, s);
    else
        attn::launch_in_proj_bwd<_Float16>(p, x, w_q, w_k, w_v, dq_cat, dk_cat, dv_cat, dw_q,
                                           dw_k, dw_v, dx, s);
    return hip_status();
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv_out, int B, int H, int n, int m,
             int d, int dv, float scale, int causal, int dtype, int flags, void* workspace,
             size_t workspace_bytes_given, void* stream) {
    Problem p;
    int st = check_problem(B, H, n, m, d, dv, scale, causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE,
                           dtype, &p);
    if (st != ATTN_OK) return st;
    if (causal && n != m) return ATTN_ECAUSAL_SHAPE;
    return attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv_out, nullptr, nullptr, B, H, n, m, d,
                       dv, scale, causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE, ATTN_LAYOUT_BHSD,
                       dtype, flags, workspace, workspace_bytes_given, stream);
}

}  // extern "C"

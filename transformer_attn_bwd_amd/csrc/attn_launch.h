// Internal interface between the C ABI (attn_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

// Element types, the values of enum attn_dtype in attn.h.
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kDtypeF16 = 2;

// Mask modes, the values of enum attn_mask in attn.h.
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;              // key j visible from row i when j <= i
constexpr int kMaskCausalBottomRight = 2;   // j <= i + m_b - n_b

struct Problem {
    long B = 0, H = 0;
    int n = 0, m = 0, d = 0, dv = 0;
    float scale = 1.f;
    bool causal = false;                    // mask != kMaskNone
    int mask = kMaskNone;
    int dtype = 0;
    const int* seqlens_q = nullptr;         // device [B] or null (n for every b)
    const int* seqlens_k = nullptr;         // device [B] or null (m for every b)
    bool bshd = false;                      // tensors [B, seq, H, dim] instead of [B, H, seq, dim]
    long heads() const { return B * H; }
};

// Tile widths the 16-bit kernels use for head widths d and dv: 64 or 128
// each (the head padded with zero columns), as 0xDDVV; 0 if d or dv is not
// a multiple of 8 in 8..128.
inline int mfma_widths(const Problem& p) {
    auto tile = [](int x) { return (x < 8 || x > 128 || x % 8) ? 0 : (x <= 64 ? 64 : 128); };
    const int td = tile(p.d), tv = tile(p.dv);
    return (td && tv) ? (td << 8) | tv : 0;
}

// What the kernels need to find a head's rows, lengths and causal offset.
struct SeqInfo {
    const int* sq;     // per-batch query lengths or null
    const int* sk;     // per-batch key lengths or null
    int H;             // heads per batch element (blockIdx.x / H is the batch)
    int br;            // 1: causal diagonal aligned bottom-right
    int bshd;          // 1: tensors are [B, seq, H, dim], else [B, H, seq, dim]
};

inline SeqInfo seq_info(const Problem& p) {
    return {p.seqlens_q, p.seqlens_k, (int)p.H, p.mask == kMaskCausalBottomRight ? 1 : 0,
            p.bshd ? 1 : 0};
}

// Workgroup order of the attention kernels, whose grids are (heads, blocks)
// with blocks per head ranked so that rank 0 is the longest under a causal
// mask.  The hardware hands the workgroups of a launch to the chip's eight
// XCDs in turn, in linear order (x fastest): rank-major order starts the
// longest blocks of every head first, and with B*H a multiple of 8 all
// blocks of a head run on one XCD.
struct TileOrder {
    int head, rank;
};
__device__ __forceinline__ TileOrder tile_order(int heads, int nblk) {
    (void)nblk;
    const int b = (int)(blockIdx.x + gridDim.x * blockIdx.y);
    return {b % heads, b / heads};
}

// Where head bh's rows live in a tensor with `rows` rows of `width`
// elements per head: element offset of its row 0, and the distance between
// consecutive rows.  [B, H, seq, dim]: the head is one contiguous block;
// [B, seq, H, dim]: rows of the H heads interleave.
struct HeadView {
    long base;
    int stride;
};
__device__ __forceinline__ HeadView head_view(const SeqInfo& si, long bh, int rows, int width) {
    if (!si.bshd) return {bh * (long)rows * width, width};
    const int b = (int)bh / si.H, h = (int)bh - b * si.H;
    return {((long)b * rows * si.H + h) * width, si.H * width};
}

// Lengths of head bh: n_b query rows and m_b key rows take part (values
// clamped into [0, n] and [0, m]); under the causal mask key j is visible
// from row i when j <= i + off.
struct SeqLens {
    int n, m, off;
};
__device__ __forceinline__ SeqLens seq_lens(const SeqInfo& si, long bh, int n, int m) {
    const int b = (int)bh / si.H;
    int nb = n, mb = m;
    if (si.sq) nb = min(max(si.sq[b], 0), n);
    if (si.sk) mb = min(max(si.sk[b], 0), m);
    return {nb, mb, si.br ? mb - nb : 0};
}

// Rows per head in the backward workspace (per-row D and rescaled LSE),
// padded so that every query tile the kernels touch is in bounds.
constexpr int kRowPad = 128;
inline int padded_rows(int n) { return (n + kRowPad - 1) / kRowPad * kRowPad; }

// dS of the stored-dS dQ mode: 16-bit tiles of 256 queries x 256 keys, one
// per query block b and key block r that the dK/dV kernel visits, each as
// eight [256 keys][32 queries] row-major blocks (one per 32-query step of
// the dK/dV kernel, 16 KB contiguous): element (key j, query i) of a tile
// at (i / 32) * 8192 + j * 32 + i % 32.  Tile (b, r) of a head sits at
// index b (b + 1) / 2 + r when `tri` (causal with the diagonal at j = i:
// the kernel visits r <= b only), else b * mblk + r.
constexpr int kDsTile = 256;
struct DsTiles {
    void* p = nullptr;       // heads * head_elems elements of the input type
    long head_elems = 0;     // elements per head (tiles * 256 * 256)
    int tri = 0;
    int mblk = 0;            // key blocks per query block (dense index)
};
inline long ds_tiles_per_head(int n, int m, bool tri) {
    const long nb = (n + kDsTile - 1) / kDsTile, mb = (m + kDsTile - 1) / kDsTile;
    return tri ? nb * (nb + 1) / 2 : nb * mb;
}

// Workspace view: lse2 [B*H][n_pad] then D [B*H][n_pad], float32; with the
// fused dQ also the float32 dQ accumulator dqacc [B*H][n_pad][acc_w], acc_w
// the 16-bit kernels' tile width for d (64 or 128).
struct Workspace {
    float* lse2;
    float* D;
    int n_pad;
    float* dqacc = nullptr;
    int acc_w = 0;
    DsTiles ds;
};

// 16-bit MFMA path, T = __bf16 or _Float16 (instantiated in the kernel
// files); return false if (d, dv) has no instantiation.
template <typename T>
bool launch_fwd_mfma(const Problem& p, const void* q, const void* k, const void* v, void* o,
                     float* lse, hipStream_t s);
template <typename T>
bool launch_bwd_preprocess_mfma(const Problem& p, const void* o, const void* dout,
                                const float* lse, const Workspace& w, hipStream_t s);
template <typename T>
bool launch_bwd_dkdv_mfma(const Problem& p, const void* q, const void* k, const void* v,
                          const void* dout, const Workspace& w, void* dk, void* dv,
                          hipStream_t s);
// With o and lse non-null the dQ pass also does the preprocess for its rows
// (same bits as launch_bwd_preprocess_mfma) and writes it to w; with them
// null it reads w.  With dqacc non-null it covers only keys j < key_limit
// and writes its unscaled float32 sums to dqacc (w.dqacc's layout) instead
// of dq.
template <typename T>
bool launch_bwd_dq_mfma(const Problem& p, const void* q, const void* k, const void* v,
                        const void* dout, const void* o, const float* lse, const Workspace& w,
                        void* dq, float* dqacc, int key_limit, hipStream_t s);
// The dK/dV kernel whose workgroups with first key >= dqa_from also add
// their dS K to w.dqacc with atomics.
template <typename T>
bool launch_bwd_dkdv_dqa_mfma(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dout, const Workspace& w, void* dk, void* dv,
                              float* dqacc, int dqa_from, hipStream_t s);
// The dK/dV kernel that also writes its dS tiles to w.ds.
template <typename T>
bool launch_bwd_dkdv_dss_mfma(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dout, const Workspace& w, void* dk, void* dv,
                              hipStream_t s);
// dq = scale * dS K from the stored tiles of w.ds.
template <typename T>
bool launch_bwd_dq_ds_mfma(const Problem& p, const void* k, const Workspace& w, void* dq,
                           hipStream_t s);
// dq = scale * w.dqacc in T.
template <typename T>
void launch_dq_convert(const Problem& p, const Workspace& w, void* dq, hipStream_t s);
// Keys per workgroup of the dK/dV kernel: the granularity of dqa_from.
constexpr int kDkdvBlock = 256;

// Projection gradients around attention (tokens as rows, T = B n):
// matrices X [T, d_model], W_Q, W_K [d_model, hd], W_V [d_model, hdv],
// W_O [hdv, d_model] with hd = H d, hdv = H dv.
struct ProjProblem {
    int T = 0, d_model = 0, hd = 0, hdv = 0;
};
template <typename T>
void launch_out_proj_bwd(const ProjProblem& p, const void* o_cat, const void* g, const void* w_o,
                         float* dw_o, void* do_cat, hipStream_t s);
template <typename T>
void launch_in_proj_bwd(const ProjProblem& p, const void* x, const void* w_q, const void* w_k,
                        const void* w_v, const void* dq_cat, const void* dk_cat,
                        const void* dv_cat, float* dw_q, float* dw_k, float* dw_v, void* dx,
                        hipStream_t s);

// fp32 path (one wave per row; any d, dv in 1..128).
bool launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o,
                    float* lse, hipStream_t s);
bool launch_bwd_preprocess_f32(const Problem& p, const float* o, const float* dout,
                               const float* lse, const Workspace& w, hipStream_t s);
bool launch_bwd_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v,
                         const float* dout, const Workspace& w, float* dk, float* dv,
                         hipStream_t s);
bool launch_bwd_dq_f32(const Problem& p, const float* q, const float* k, const float* v,
                       const float* dout, const Workspace& w, float* dq, hipStream_t s);

}  // namespace attn

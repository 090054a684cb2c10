// Float32 attention forward and backward for any head widths 1..128.
//
// This path exists for full-precision checks, not for speed: one wave per
// row, lanes spread across the head dimension (two elements per lane at
// most), dot products reduced across the wave.  The formulas are the same
// as the 16-bit path's (mlgrind "Forward"/"Backward"; eulerpad P2-P6), with
// natural-base exponentials and float32 everywhere, and so are the
// per-batch lengths and causal offsets: rows i < nb and keys j < mb take
// part, key j is visible from row i when j <= i + off (causal), rows past
// nb or with no visible key get O = 0, LSE = -inf, dQ = 0, keys past mb get
// dK = dV = 0.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int E = 2;   // elements per lane: 64 lanes x 2 = 128 columns

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

struct RowVec {
    float x[E];
    __device__ __forceinline__ void load(const float* p, int len, int lane) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            x[e] = c < len ? p[c] : 0.f;
        }
    }
    __device__ __forceinline__ float dot(const float* p, int len, int lane) const {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            if (c < len) acc += x[e] * p[c];
        }
        return wave_sum(acc);
    }
    __device__ __forceinline__ void store(float* p, int len, int lane, float mult) const {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            if (c < len) p[c] = x[e] * mult;
        }
    }
};

// One wave per query row: online softmax over the visible keys.
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      float* __restrict__ o,
                                                      float* __restrict__ lse, int n, int m,
                                                      int d, int dv, float scale, int causal,
                                                      SeqInfo si) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const long bh = blockIdx.y;
    if (i >= n) return;
    const SeqLens len = seq_lens(si, bh, n, m);
    const HeadView hq = head_view(si, bh, n, d), hk = head_view(si, bh, m, d);
    const HeadView hv = head_view(si, bh, m, dv), ho = head_view(si, bh, n, dv);
    const float* kh = k + hk.base;
    const float* vh = v + hv.base;
    RowVec qi, acc;
    qi.load(q + hq.base + (long)i * hq.stride, d, lane);
#pragma unroll
    for (int e = 0; e < E; ++e) acc.x[e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    int jend = causal ? min(i + len.off + 1, len.m) : len.m;
    if (i >= len.n) jend = 0;
    for (int j = 0; j < jend; ++j) {
        const float s = qi.dot(kh + (long)j * hk.stride, d, lane) * scale;
        const float m_new = fmaxf(m_run, s);
        const float alpha = expf(m_run - m_new);
        const float p = expf(s - m_new);
        l_run = l_run * alpha + p;
        const float* vj = vh + (long)j * hv.stride;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            acc.x[e] = acc.x[e] * alpha + (c < dv ? p * vj[c] : 0.f);
        }
        m_run = m_new;
    }
    const bool seen = jend > 0;
    acc.store(o + ho.base + (long)i * ho.stride, dv, lane, seen ? 1.f / l_run : 0.f);
    if (lane == 0) lse[bh * (long)n + i] = seen ? m_run + logf(l_run) : -INFINITY;
}

// One thread per row: D_i = dO_i . O_i; LSE copied (natural base) into the
// workspace.  Padded rows and rows that saw no key get LSE = +inf, so that
// their P is exactly 0, and D = 0.
__global__ __launch_bounds__(256) void preprocess_f32_kernel(
    const float* __restrict__ o, const float* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ lse_ws, float* __restrict__ Dw, int n, int n_pad, int dv,
    long total_rows, SeqInfo si) {
    const long row = (long)blockIdx.x * 256 + threadIdx.x;
    if (row >= total_rows) return;
    const long bh = row / n_pad;
    const int i = (int)(row % n_pad);
    const int nb = seq_lens(si, bh, n, 1).n;
    float acc = 0.f, l = -INFINITY;
    if (i < nb) {
        const HeadView ho = head_view(si, bh, n, dv);
        const float* orow = o + ho.base + (long)i * ho.stride;
        const float* drow = dout + ho.base + (long)i * ho.stride;
        for (int c = 0; c < dv; ++c) acc += orow[c] * drow[c];
        l = lse[bh * (long)n + i];
    }
    lse_ws[row] = l > -INFINITY ? l : INFINITY;
    Dw[row] = acc;
}

// One wave per key row j: dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij Q_i.
__global__ __launch_bounds__(256) void dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse_ws,
    const float* __restrict__ Dw, float* __restrict__ dk, float* __restrict__ dvo, int n, int m,
    int d, int dv, int n_pad, float scale, int causal, SeqInfo si) {
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    const long bh = blockIdx.y;
    if (j >= m) return;
    const SeqLens len = seq_lens(si, bh, n, m);
    const HeadView hq = head_view(si, bh, n, d), hk = head_view(si, bh, m, d);
    const HeadView hv = head_view(si, bh, m, dv), ho = head_view(si, bh, n, dv);
    const float* qh = q + hq.base;
    const float* oh = dout + ho.base;
    RowVec kj, vj, gk, gv;
    kj.load(k + hk.base + (long)j * hk.stride, d, lane);
    vj.load(v + hv.base + (long)j * hv.stride, dv, lane);
#pragma unroll
    for (int e = 0; e < E; ++e) gk.x[e] = gv.x[e] = 0.f;
    const int iend = j < len.m ? len.n : 0;
    for (int i = causal ? max(j - len.off, 0) : 0; i < iend; ++i) {
        const float* qi = qh + (long)i * hq.stride;
        const float* doi = oh + (long)i * ho.stride;
        const float s = kj.dot(qi, d, lane) * scale;
        const float p = expf(s - lse_ws[bh * (long)n_pad + i]);
        const float dp = vj.dot(doi, dv, lane);
        const float ds = p * (dp - Dw[bh * (long)n_pad + i]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            if (c < d) gk.x[e] += ds * qi[c];
            if (c < dv) gv.x[e] += p * doi[c];
        }
    }
    gk.store(dk + hk.base + (long)j * hk.stride, d, lane, scale);
    gv.store(dvo + hv.base + (long)j * hv.stride, dv, lane, 1.f);
}

// One wave per query row i: dQ_i = scale sum_j dS_ij K_j.
__global__ __launch_bounds__(256) void dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse_ws,
    const float* __restrict__ Dw, float* __restrict__ dq, int n, int m, int d, int dv, int n_pad,
    float scale, int causal, SeqInfo si) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const long bh = blockIdx.y;
    if (i >= n) return;
    const SeqLens len = seq_lens(si, bh, n, m);
    const HeadView hq = head_view(si, bh, n, d), hk = head_view(si, bh, m, d);
    const HeadView hv = head_view(si, bh, m, dv), ho = head_view(si, bh, n, dv);
    const float* kh = k + hk.base;
    const float* vh = v + hv.base;
    RowVec qi, doi, g;
    qi.load(q + hq.base + (long)i * hq.stride, d, lane);
    doi.load(dout + ho.base + (long)i * ho.stride, dv, lane);
#pragma unroll
    for (int e = 0; e < E; ++e) g.x[e] = 0.f;
    const float li = lse_ws[bh * (long)n_pad + i];
    const float Di = Dw[bh * (long)n_pad + i];
    int jend = causal ? min(i + len.off + 1, len.m) : len.m;
    if (i >= len.n || li == INFINITY) jend = 0;
    for (int j = 0; j < jend; ++j) {
        const float* kj = kh + (long)j * hk.stride;
        const float s = qi.dot(kj, d, lane) * scale;
        const float p = expf(s - li);
        const float dp = doi.dot(vh + (long)j * hv.stride, dv, lane);
        const float ds = p * (dp - Di);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            if (c < d) g.x[e] += ds * kj[c];
        }
    }
    g.store(dq + hq.base + (long)i * hq.stride, d, lane, scale);
}

}  // namespace

bool launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o,
                    float* lse, hipStream_t s) {
    if (p.d > 64 * E || p.dv > 64 * E) return false;
    dim3 grid((unsigned)((p.n + 3) / 4), (unsigned)p.heads());
    fwd_f32_kernel<<<grid, 256, 0, s>>>(q, k, v, o, lse, p.n, p.m, p.d, p.dv, p.scale,
                                        p.causal ? 1 : 0, seq_info(p));
    return true;
}

bool launch_bwd_preprocess_f32(const Problem& p, const float* o, const float* dout,
                               const float* lse, const Workspace& w, hipStream_t s) {
    const long total = p.heads() * (long)w.n_pad;
    preprocess_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
        o, dout, lse, w.lse2, w.D, p.n, w.n_pad, p.dv, total, seq_info(p));
    return true;
}

bool launch_bwd_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v,
                         const float* dout, const Workspace& w, float* dk, float* dv,
                         hipStream_t s) {
    if (p.d > 64 * E || p.dv > 64 * E) return false;
    dim3 grid((unsigned)((p.m + 3) / 4), (unsigned)p.heads());
    dkdv_f32_kernel<<<grid, 256, 0, s>>>(q, k, v, dout, w.lse2, w.D, dk, dv, p.n, p.m, p.d,
                                         p.dv, w.n_pad, p.scale, p.causal ? 1 : 0, seq_info(p));
    return true;
}

bool launch_bwd_dq_f32(const Problem& p, const float* q, const float* k, const float* v,
                       const float* dout, const Workspace& w, float* dq, hipStream_t s) {
    if (p.d > 64 * E || p.dv > 64 * E) return false;
    dim3 grid((unsigned)((p.n + 3) / 4), (unsigned)p.heads());
    dq_f32_kernel<<<grid, 256, 0, s>>>(q, k, v, dout, w.lse2, w.D, dq, p.n, p.m, p.d, p.dv,
                                       w.n_pad, p.scale, p.causal ? 1 : 0, seq_info(p));
    return true;
}

}  // namespace attn

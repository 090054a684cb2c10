// Backward attention on 16-bit MFMA (bf16 or f16 inputs, float32
// accumulation): the preprocess kernel and the dK/dV kernel without fused
// dQ work (the kernel itself is in attn_bwd_dkdv.h, the dQ pass in
// attn_bwd_dq_mfma.hip).
//
// Preprocess: D_i = rowsum(dO o O)_i, the cheap form of rowsum(dP o P)
// (step-by-step derivation, "Gradient of S"; mlgrind "Follow-up"), stored
// negated (the dK/dV kernel starts its dP accumulators from -D, so that
// dS = P o (dP - D) is one multiply), and LSE rescaled to base 2 so that
// P = exp2(S * scale * log2e - LSE2).
#include "attn_bwd_dkdv.h"

namespace attn {
namespace {

// ---------------------------------------------------------------- preprocess

template <typename T, int DV>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(
    const T* __restrict__ o, const T* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ lse2, float* __restrict__ Dw, int n, int dvg, int n_pad,
    long total_rows, SeqInfo si) {
    constexpr int LPR = DV / 8;        // lanes per row, 8 elements (16 bytes) each
    constexpr int RPB = 256 / LPR;     // rows per block
    const int tid = threadIdx.x;
    const long row = (long)blockIdx.x * RPB + tid / LPR;
    const int part = tid % LPR;
    const bool valid_row = row < total_rows;
    const long bh = valid_row ? row / n_pad : 0;
    const int i = valid_row ? (int)(row % n_pad) : 0;
    const int nb = seq_lens(si, bh, n, 1).n;
    float acc = 0.f;
    // rows hold dvg <= DV elements; lanes past them add nothing.  Explicit
    // fused multiply-adds, one per element in order: the dQ pass repeats
    // this sum and must get the same bits (left to itself the compiler pairs
    // fp16 products into dot2 instructions here but not there).
    if (valid_row && i < nb && 8 * part < dvg) {
        const HeadView hv = head_view(si, bh, n, dvg);
        const long off = hv.base + (long)i * hv.stride + 8 * part;
        vec8<T> a = gload8(o + off);
        vec8<T> b = gload8(dout + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    // Rows past nb, and rows that saw no key (LSE = -inf), get LSE2 = +inf
    // so that every P of theirs is exactly 0.
    if (valid_row && part == 0) {
        const float l = i < nb ? lse[bh * (long)n + i] : -INFINITY;
        lse2[row] = l > -INFINITY ? l * kLog2e : INFINITY;
        Dw[row] = -acc;
    }
}

template <typename T, int DV>
void launch_pre(const Problem& p, const void* o, const void* dout, const float* lse,
                const Workspace& w, hipStream_t s) {
    constexpr int RPB = 256 / (DV / 8);
    const long total = p.heads() * (long)w.n_pad;
    const unsigned blocks = (unsigned)((total + RPB - 1) / RPB);
    bwd_preprocess_kernel<T, DV><<<blocks, 256, 0, s>>>((const T*)o, (const T*)dout, lse,
                                                        w.lse2, w.D, p.n, p.dv, w.n_pad, total,
                                                        seq_info(p));
}

}  // namespace

template <typename T>
bool launch_bwd_preprocess_mfma(const Problem& p, const void* o, const void* dout,
                                const float* lse, const Workspace& w, hipStream_t s) {
    switch (mfma_widths(p) & 0xff) {
    case 0x40: launch_pre<T, 64>(p, o, dout, lse, w, s); break;
    case 0x80: launch_pre<T, 128>(p, o, dout, lse, w, s); break;
    default: return false;
    }
    return true;
}

template <typename T>
bool launch_bwd_dkdv_mfma(const Problem& p, const void* q, const void* k, const void* v,
                          const void* dout, const Workspace& w, void* dk, void* dv,
                          hipStream_t s) {
    switch (mfma_widths(p)) {
    case 0x4040: launch_dkdv<T, 64, 64, false>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    case 0x4080: launch_dkdv<T, 64, 128, false>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    case 0x8040: launch_dkdv<T, 128, 64, false>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    case 0x8080: launch_dkdv<T, 128, 128, false>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    default: return false;
    }
    return true;
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template bool launch_bwd_preprocess_mfma<ATTN_ELEM>(const Problem&, const void*, const void*,
                                                   const float*, const Workspace&, hipStream_t);
template bool launch_bwd_dkdv_mfma<ATTN_ELEM>(const Problem&, const void*, const void*,
                                             const void*, const void*, const Workspace&, void*,
                                             void*, hipStream_t);

}  // namespace attn

// Backward attention on 16-bit MFMA (bf16 or f16 inputs, float32
// accumulation): the preprocess and dK/dV kernels (the dQ pass is in
// attn_bwd_dq_mfma.hip).
//
//  1. preprocess: D_i = rowsum(dO o O)_i, the cheap form of rowsum(dP o P)
//     (step-by-step derivation, "Gradient of S"; mlgrind "Follow-up"), and
//     LSE rescaled to base 2 so that P = exp2(S * scale * log2e - LSE2).
//  2. dK/dV: one workgroup per 256 keys of a head (64 per wave); it walks
//     the query tiles, recomputes S = Q K^T and P, and accumulates
//     dV += P^T dO and dK += dS^T Q in registers (eulerpad P2, P6).
//
// In kernel 2 the lane owns a key: the accumulator layout of S (rows =
// queries, columns = keys) is exactly the A-operand layout P^T and dS^T
// need (rows = keys, k = queries), so P and dS never leave registers; the
// partners dO and Q are read with transposing LDS reads in the matching
// row-of-C order.
// The causal mask (S_ij = -inf for j > i, i.e. P_ij = 0, eulerpad P8) is
// applied only in tiles that straddle the diagonal; tiles entirely above
// it are never visited.
#include "attn_device.h"
#include "attn_launch.h"

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
        Dw[row] = acc;
    }
}

// ---------------------------------------------------------------- dK / dV

template <int D, int DV>
struct DkdvCfg {
    static constexpr int NW = 4;             // waves per workgroup
    static constexpr int KW = 64;            // keys per wave (two 32-key MFMA tiles)
    static constexpr int BN = NW * KW;       // keys per workgroup
    static constexpr int BM = 32;            // queries per step
    static constexpr int LA = 4;             // operand reads issued this many MFMAs ahead
};

// Per-step schedule of the dK/dV kernel, all compile-time.  With KA = D/16,
// KB = DV/16, NX = D/32, NXV = DV/32 the step issues, in order,
//   S    2KA MFMAs  j = 2r + kt          S[kt]  += Q_r  K[kt]_r^T
//   dP   2KB MFMAs  j = 2KA + 2r + kt    dP[kt] += dO_r V[kt]_r^T
//   dV  4NXV MFMAs  2(c NXV + x) + kt    dV[kt][x]^T += (dO_c,x)^T P[kt]_c
//   dK  4NX  MFMAs  2(c NX + x) + kt     dK[kt][x]^T += (Q_c,x)^T dS[kt]_c
// (kt: 32-key tile of the wave, r: 16-wide chunk of d or dv, c: 16-query
// half of the step, x: 32-column block).  Operand fragments read from LDS:
//   f <  KA               Q rows, chunk f              (first used by j = 2f)
//   f < 3KA               K rows of tile kt, chunk r   (j = 2r + kt)
//   f < 3KA + KB          dO rows, chunk r             (j = 2KA + 2r)
//   f < 3KA + KB + 2NXV   dO^T half c, block x         (dV, first j of (c, x))
//   f < 3KA + KB + 2NXV + 2NX   Q^T half c, block x    (dK, first j of (c, x))
template <int D, int DV>
struct DkdvSched {
    static constexpr int KA = D / 16, KB = DV / 16, NX = D / 32, NXV = DV / 32;
    static constexpr int J_DP = 2 * KA, J_DV = J_DP + 2 * KB, J_DK = J_DV + 4 * NXV;
    static constexpr int NJ = J_DK + 4 * NX;
    static constexpr int F_K = KA, F_DO = 3 * KA, F_DOT = F_DO + KB, F_QT = F_DOT + 2 * NXV;
    static constexpr int NF = F_QT + 2 * NX;
    static constexpr int first_use(int f) {
        if (f < F_K) return 2 * f;
        if (f < F_DO) return 2 * ((f - F_K) % KA) + (f - F_K) / KA;
        if (f < F_DOT) return J_DP + 2 * (f - F_DO);
        if (f < F_QT) return J_DV + 2 * (f - F_DOT);
        return J_DK + 2 * (f - F_QT);
    }
    static constexpr int issue_at(int f, int la) {
        return first_use(f) - la < 0 ? 0 : first_use(f) - la;
    }
    // Softmax elements, 32 per step per lane: element i is accumulator
    // slot e(i) of key tile kt(i); ordered by 8-slot operand chunk, so
    // that each 16-bit operand is complete early.
    static constexpr int elem_c(int i) { return i / 16; }
    static constexpr int elem_kt(int i) { return (i / 8) % 2; }
    static constexpr int elem_e(int i) { return 8 * elem_c(i) + i % 8; }
    // P = exp2(...) of element i is formed in dP slot p_slot(i), dS in dV
    // slot ds_slot(i).
    static constexpr int p_slot(int i) { return J_DP + (i * 2 * KB) / 32; }
    static constexpr int ds_slot(int i) { return J_DV + (i * 4 * NXV) / 32; }
    // statistics of row group vq (accumulator slots 4vq..4vq+3) are read
    // two slots before the first element that needs them
    static constexpr int first_elem_of_vq(int vq) { return 16 * (vq / 2) + 4 * (vq % 2); }
    static constexpr int l_slot(int vq) { return p_slot(first_elem_of_vq(vq)) - 2; }
    static constexpr int d_slot(int vq) { return ds_slot(first_elem_of_vq(vq)) - 2; }
};

// One workgroup per 256 keys of a head, four waves of 64 keys.  The
// workgroup's K rows sit in LDS for the whole kernel and this wave's V rows
// in registers (B operands of S = Q K^T and dP = dO V^T, lane = key); the
// query tiles (32 rows of Q and dO, with their LSE2 and D) stream through
// two LDS buffers.  Each Q, dO, Q^T and dO^T fragment read from LDS feeds
// two MFMAs (the wave's two key tiles).  dK and dV accumulate, transposed,
// in AGPRs: the A and B operands of a 32x32x16 MFMA have the same lane
// layout, so swapping them yields the transposed product in the same
// registers, and the transposed tiles hold four consecutive columns of one
// key per lane group, which the epilogue needs.
template <typename T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ Dw, T* __restrict__ dk, T* __restrict__ dvo, int n, int m,
    int dg, int dvg, int n_pad, float scale, float c2, SeqInfo si) {
    using C = DkdvCfg<D, DV>;
    using SC = DkdvSched<D, DV>;
    constexpr int BM = C::BM, NW = C::NW, LA = C::LA;
    // One LDS variable per buffer: the compiler can then tell that reads
    // of one buffer do not alias the asynchronous fills of the other, and
    // does not make them wait for those fills.
    __shared__ __align__(1024) T sK[C::BN * D];
    __shared__ __align__(1024) T sQ0[BM * D];
    __shared__ __align__(1024) T sQ1[BM * D];
    __shared__ __align__(1024) T sO0[BM * DV];
    __shared__ __align__(1024) T sO1[BM * DV];
    __shared__ __align__(256) float sL0[64];
    __shared__ __align__(256) float sL1[64];
    __shared__ __align__(256) float sD0[64];
    __shared__ __align__(256) float sD1[64];
    auto pick = [](auto b_, auto* x0, auto* x1) __attribute__((always_inline)) {
        if constexpr (decltype(b_)::value == 0) return x0;
        else return x1;
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const long bh = blockIdx.x;
    const int j0 = blockIdx.y * C::BN;
    const int kw0 = j0 + C::KW * wave;      // this wave's first key
    // This head's query and key lengths and causal offset: rows i < nb take
    // part, keys j < mb, and key j is visible from row i when j <= i + off.
    const SeqLens len = seq_lens(si, bh, n, m);
    const int nb = len.n, mb = len.m, off = len.off;

    // Rows of Q and K hold dg <= D elements, rows of V and dO dvg <= DV (each
    // a multiple of 8); the columns past them are zeros in registers and
    // LDS, so they add nothing to any product.
    const HeadView hq = head_view(si, bh, n, dg), hk = head_view(si, bh, m, dg);
    const HeadView hv = head_view(si, bh, m, dvg), ho = head_view(si, bh, n, dvg);
    const T* qh = q + hq.base;
    const T* kh = k + hk.base;
    const T* vh = v + hv.base;
    const T* oh = dout + ho.base;
    const float* lh = lse2 + bh * (long)n_pad;
    const float* dh = Dw + bh * (long)n_pad;

    // K rows j0 .. j0+255 into LDS (rows past mb read as zeros: their S and
    // P only reach dK and dV rows that are written as zeros).
    {
        TileLoader<D, C::BN, NW> ldK;
        ldK.init(wave, lane, dg, hk.stride);
        tile_fill<D, C::BN, NW>(ldK, sK, make_rsrc(kh, (uint32_t)mb * hk.stride * 2), j0, wave);
    }
    // This lane's V row for key tile kt (key kw0 + 32 kt + li): B operand of
    // dP = dO V^T.
    vec8<T> vreg[2][DV / 16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const int key = kw0 + 32 * kt + li;
#pragma unroll
        for (int kc = 0; kc < DV / 16; ++kc)
            vreg[kt][kc] = (key < mb && 16 * kc + 8 * g < dvg)
                               ? gload8(vh + (long)key * hv.stride + 16 * kc + 8 * g)
                               : vec8<T>{};
    }

    TileOffsets<D> toQ;
    toQ.init(lane);
    TileOffsets<DV> toO;
    toO.init(lane);
    const T* Kw = sK + C::KW * wave * D;  // this wave's 64 K rows

    // Causal: rows below j0 - off see none of the workgroup's keys; query
    // tiles that start below its last key minus off straddle the diagonal
    // and are masked, the rest see every key of the workgroup.  The masked
    // run is made even unless it covers every step, so that the plain loop
    // starts on buffer 0.
    const int i_begin = CAUSAL ? max(j0 - off, 0) / BM * BM : 0;
    const int i_end = (nb + BM - 1) / BM * BM;
    const int nsteps = (j0 < mb && i_end > i_begin) ? (i_end - i_begin) / BM : 0;
    int n_masked = 0;
    if (CAUSAL) {
        n_masked = min(max((j0 + C::BN - 1 - off - i_begin + BM - 1) / BM, 0), nsteps);
        if (n_masked < nsteps) n_masked = min((n_masked + 1) & ~1, nsteps);
    }

    // Query tile i0 into a buffer: Q and dO rows (rows past nb come back as
    // zeros; their LSE2 is +inf, so P = 0 and they contribute nothing), and
    // the per-row LSE2 and D.
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(qh, (uint32_t)nb * hq.stride * 2);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(oh, (uint32_t)nb * ho.stride * 2);
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(lh, (uint32_t)n_pad * 4);
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(dh, (uint32_t)n_pad * 4);
    TileLoader<D, BM, NW> ldQ;
    ldQ.init(wave, lane, dg, hq.stride);
    TileLoader<DV, BM, NW> ldO;
    ldO.init(wave, lane, dvg, ho.stride);
    auto stage = [&](auto buf_, int i0) __attribute__((always_inline)) {
        tile_fill<D, BM, NW>(ldQ, pick(buf_, sQ0, sQ1), rQ, i0, wave);
        tile_fill<DV, BM, NW>(ldO, pick(buf_, sO0, sO1), rO, i0, wave);
        if (wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (ATTN_LDS void*)pick(buf_, sL0, sL1), 4,
                                                     4 * lane, 4 * i0, 0, 0);
        else if (wave == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (ATTN_LDS void*)pick(buf_, sD0, sD1), 4,
                                                     4 * lane, 4 * i0, 0, 0);
    };

    f32x16 accK[2][D / 32], accV[2][DV / 32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int x = 0; x < D / 32; ++x) accK[kt][x] = zero16();
#pragma unroll
        for (int x = 0; x < DV / 32; ++x) accV[kt][x] = zero16();
    }

    // One query tile: the SC schedule, one MFMA per slot, fenced with
    // sched_barrier so that the operand reads (LA slots ahead), the matrix
    // products and the softmax work interleave as written.  MASKED steps
    // apply the causal mask.
    auto compute = [&](auto buf_, auto masked_, int i0) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_)::value;
        const T* Qs = pick(buf_, sQ0, sQ1);
        const T* Os = pick(buf_, sO0, sO1);
        const float* Ls = pick(buf_, sL0, sL1);
        const float* Ds = pick(buf_, sD0, sD1);

        auto load_frag = [&](auto f_) __attribute__((always_inline)) -> vec8<T> {
            constexpr int f = decltype(f_)::value;
            if constexpr (f < SC::F_K) {
                return tile_read8_at<D>(Qs, toQ, 0, f);
            } else if constexpr (f < SC::F_DO) {
                constexpr int kt = (f - SC::F_K) / SC::KA, r = (f - SC::F_K) % SC::KA;
                return tile_read8_at<D>(Kw, toQ, 32 * kt, r);
            } else if constexpr (f < SC::F_DOT) {
                return tile_read8_at<DV>(Os, toO, 0, f - SC::F_DO);
            } else if constexpr (f < SC::F_QT) {
                constexpr int c = (f - SC::F_DOT) / SC::NXV, x = (f - SC::F_DOT) % SC::NXV;
                return tile_read_tr_at<DV>(Os, toO, 16 * c, x);
            } else {
                constexpr int c = (f - SC::F_QT) / SC::NX, x = (f - SC::F_QT) % SC::NX;
                return tile_read_tr_at<D>(Qs, toQ, 16 * c, x);
            }
        };

        f32x16 S[2], dP[2];          // S is overwritten by P
        vec8<T> Pb[2][2], dSb[2][2];
        f32x4 l4[4], d4[4];
        vec8<T> fr[SC::NF];

        // Query of accumulator slot e: i0 + 8(e>>2) + 4g + (e&3); key of
        // tile kt: kw0 + 32kt + li.  The slot is masked when key > query,
        // i.e. when 8(e>>2) + (e&3) < lim[kt].
        int lim[2];
        if constexpr (MASKED) {
            lim[0] = kw0 + li - off - i0 - 4 * g;
            lim[1] = lim[0] + 32;
        }

        auto p_elem = [&](auto i_) __attribute__((always_inline)) {
            constexpr int i = decltype(i_)::value;
            constexpr int kt = SC::elem_kt(i), e = SC::elem_e(i), vq = e >> 2, r = e & 3;
            float pv = fast_exp2(__builtin_fmaf(S[kt][e], c2, -l4[vq][r]));
            if constexpr (MASKED) pv = (8 * vq + r < lim[kt]) ? 0.f : pv;
            S[kt][e] = pv;
            if constexpr (i % 8 == 7) {
                constexpr int c = SC::elem_c(i), b = 8 * c;
                Pb[kt][c] = pack8<T>(S[kt][b], S[kt][b + 1], S[kt][b + 2], S[kt][b + 3], S[kt][b + 4],
                                  S[kt][b + 5], S[kt][b + 6], S[kt][b + 7]);
            }
        };
        auto ds_elem = [&](auto i_) __attribute__((always_inline)) {
            constexpr int i = decltype(i_)::value;
            constexpr int kt = SC::elem_kt(i), e = SC::elem_e(i), vq = e >> 2, r = e & 3;
            dP[kt][e] = S[kt][e] * (dP[kt][e] - d4[vq][r]);
            if constexpr (i % 8 == 7) {
                constexpr int c = SC::elem_c(i), b = 8 * c;
                dSb[kt][c] = pack8<T>(dP[kt][b], dP[kt][b + 1], dP[kt][b + 2], dP[kt][b + 3],
                                   dP[kt][b + 4], dP[kt][b + 5], dP[kt][b + 6], dP[kt][b + 7]);
            }
        };

        static_for<SC::NF>([&](auto f_) {
            constexpr int f = decltype(f_)::value;
            if constexpr (SC::issue_at(f, LA) == 0) fr[f] = load_frag(f_);
        });
        __builtin_amdgcn_sched_barrier(0);

        static_for<SC::NJ>([&](auto j_) {
            constexpr int j = decltype(j_)::value;
            // operand reads for later slots
            static_for<SC::NF>([&](auto f_) {
                constexpr int f = decltype(f_)::value;
                if constexpr (j > 0 && SC::issue_at(f, LA) == j) fr[f] = load_frag(f_);
            });
            // statistics
            static_for<4>([&](auto vq_) {
                constexpr int vq = decltype(vq_)::value;
                if constexpr (SC::l_slot(vq) == j)
                    l4[vq] = *reinterpret_cast<const f32x4*>(Ls + 8 * vq + 4 * g);
                if constexpr (SC::d_slot(vq) == j)
                    d4[vq] = *reinterpret_cast<const f32x4*>(Ds + 8 * vq + 4 * g);
            });
            // the product of this slot
            constexpr int kt = j % 2;
            if constexpr (j < SC::J_DP) {
                constexpr int r = j / 2;
                if constexpr (r == 0) S[kt] = zero16();
                S[kt] = mfma32(fr[r], fr[SC::F_K + kt * SC::KA + r], S[kt]);
            } else if constexpr (j < SC::J_DV) {
                constexpr int r = (j - SC::J_DP) / 2;
                if constexpr (r == 0) dP[kt] = zero16();
                dP[kt] = mfma32(fr[SC::F_DO + r], vreg[kt][r], dP[kt]);
            } else if constexpr (j < SC::J_DK) {
                constexpr int cx = (j - SC::J_DV) / 2, c = cx / SC::NXV, x = cx % SC::NXV;
                mfma32_agpr(fr[SC::F_DOT + cx], Pb[kt][c], accV[kt][x]);
            } else {
                constexpr int cx = (j - SC::J_DK) / 2, c = cx / SC::NX, x = cx % SC::NX;
                mfma32_agpr(fr[SC::F_QT + cx], dSb[kt][c], accK[kt][x]);
            }
            // softmax work of this slot
            static_for<32>([&](auto i_) {
                constexpr int i = decltype(i_)::value;
                if constexpr (SC::p_slot(i) == j) p_elem(i_);
                if constexpr (SC::ds_slot(i) == j) ds_elem(i_);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    auto do_step = [&](auto buf_, auto masked_, int s) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_)::value;
        const int i0 = i_begin + s * BM;
        if (s + 1 < nsteps) stage(std::integral_constant<int, buf ^ 1>{}, i0 + BM);
        compute(buf_, masked_, i0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using MaskOn = std::integral_constant<bool, true>;
    using MaskOff = std::integral_constant<bool, false>;

    if (nsteps > 0) stage(B0{}, i_begin);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Step s uses buffer s & 1; the masked run has an even length unless it
    // covers every step, so the plain loop starts on buffer 0.
    int s = 0;
    for (; s + 1 < n_masked; s += 2) {
        do_step(B0{}, MaskOn{}, s);
        do_step(B1{}, MaskOn{}, s + 1);
    }
    if (s < n_masked) do_step(B0{}, MaskOn{}, s++);
    for (; s + 1 < nsteps; s += 2) {
        do_step(B0{}, MaskOff{}, s);
        do_step(B1{}, MaskOff{}, s + 1);
    }
    if (s < nsteps) do_step(B0{}, MaskOff{}, s);

    // wait states between the last MFMA writing an accumulator and the
    // reads below
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // The products were taken with the operands swapped, so the
    // accumulators hold dK^T and dV^T: slot vv of tile (kt, x) is column
    // 32x + 8(vv>>2) + 4g + (vv&3) of key kw0 + 32kt + li.  They go out
    // through this wave's 64 rows of the K tile in LDS (no other wave reads
    // them, and the last step's barrier has passed): each slab of D columns
    // is written there row-major (16-byte chunks XOR-swizzled by row), read
    // back as whole rows and stored 16 bytes per lane, 1 KB of contiguous
    // rows per instruction.  Keys past mb are padding: zeros, selected rather
    // than multiplied, since a padded key's accumulators may hold inf (S = 0
    // there, and P = exp2(-LSE2) overflows when a row's LSE is very
    // negative).
    T* reg = sK + C::KW * wave * D;
    auto put_tile = [&](auto W_, const f32x16 (&acc)[2][W_.value / 32], int wcols, float mult,
                        T* out, long stride) __attribute__((always_inline)) {
        constexpr int W = decltype(W_)::value;
        constexpr int SW = W < D ? W : D;      // slab width: what the region holds
        constexpr int CH = SW / 8;             // 16-byte chunks per slab row
#pragma unroll
        for (int sl = 0; sl < W / SW; ++sl) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int row = 32 * kt + li;
                const bool real = kw0 + row < mb;
#pragma unroll
                for (int xs = 0; xs < SW / 32; ++xs) {
                    const int x = sl * (SW / 32) + xs;
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        vec4<T> w4;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w4[r] = real ? (T)(acc[kt][x][4 * vq + r] * mult) : (T)0.f;
                        const int chunk = 4 * xs + vq;
                        *reinterpret_cast<vec4<T>*>(
                            reg + row * SW + 8 * (chunk ^ (row & (CH - 1))) + 4 * g) = w4;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int lin = 64 * i + lane, row = lin / CH, chunk = lin % CH;
                const vec8<T> w8 = *reinterpret_cast<const vec8<T>*>(
                    reg + row * SW + 8 * (chunk ^ (row & (CH - 1))));
                const int key = kw0 + row, col = sl * SW + 8 * chunk;
                if (key < m && col < wcols)
                    *reinterpret_cast<vec8<T>*>(out + (long)key * stride + col) = w8;
            }
        }
    };
    put_tile(std::integral_constant<int, D>{}, accK, dg, scale, dk + hk.base, hk.stride);
    put_tile(std::integral_constant<int, DV>{}, accV, dvg, 1.f, dvo + hv.base, hv.stride);
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

template <typename T, int D, int DV>
void launch_dkdv(const Problem& p, const void* q, const void* k, const void* v,
                 const void* dout, const Workspace& w, void* dk, void* dv, hipStream_t s) {
    using C = DkdvCfg<D, DV>;
    dim3 grid((unsigned)p.heads(), (unsigned)((p.m + C::BN - 1) / C::BN));
    const float c2 = p.scale * kLog2e;
    const SeqInfo si = seq_info(p);
    if (p.causal)
        bwd_dkdv_kernel<T, D, DV, true><<<grid, 256, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (const T*)dout, w.lse2, w.D,
            (T*)dk, (T*)dv, p.n, p.m, p.d, p.dv, w.n_pad, p.scale, c2, si);
    else
        bwd_dkdv_kernel<T, D, DV, false><<<grid, 256, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (const T*)dout, w.lse2, w.D,
            (T*)dk, (T*)dv, p.n, p.m, p.d, p.dv, w.n_pad, p.scale, c2, si);
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
    case 0x4040: launch_dkdv<T, 64, 64>(p, q, k, v, dout, w, dk, dv, s); break;
    case 0x4080: launch_dkdv<T, 64, 128>(p, q, k, v, dout, w, dk, dv, s); break;
    case 0x8040: launch_dkdv<T, 128, 64>(p, q, k, v, dout, w, dk, dv, s); break;
    case 0x8080: launch_dkdv<T, 128, 128>(p, q, k, v, dout, w, dk, dv, s); break;
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

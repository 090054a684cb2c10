// Backward attention on bf16 MFMA (float32 accumulation): the preprocess
// and dK/dV kernels (the dQ pass is in attn_bwd_dq_bf16.hip).
//
//  1. preprocess: D_i = rowsum(dO o O)_i, the cheap form of rowsum(dP o P)
//     (step-by-step derivation, "Gradient of S"; mlgrind "Follow-up"), and
//     LSE rescaled to base 2 so that P = exp2(S * scale * log2e - LSE2).
//  2. dK/dV: one workgroup per 128 keys of a head (32 per wave); it walks
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

// Order of the S and dP products within a query (or key) half: the two
// accumulation chains alternate so that consecutive products never depend
// on each other; the longer chain's remainder goes last.
template <int KA, int KB>
constexpr int a_order(int r0) {
    constexpr int m = KA < KB ? KA : KB;
    if (r0 < 2 * m) return (r0 & 1) ? KA + r0 / 2 : r0 / 2;
    return KA > KB ? (r0 - m) : (KA + (r0 - m));
}

// ---------------------------------------------------------------- preprocess

template <int DV>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(
    const bf16* __restrict__ o, const bf16* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ lse2, float* __restrict__ Dw, int n, int n_pad, long total_rows) {
    constexpr int LPR = DV / 8;        // lanes per row, 8 elements (16 bytes) each
    constexpr int RPB = 256 / LPR;     // rows per block
    const int tid = threadIdx.x;
    const long row = (long)blockIdx.x * RPB + tid / LPR;
    const int part = tid % LPR;
    const bool valid_row = row < total_rows;
    const long bh = valid_row ? row / n_pad : 0;
    const int i = valid_row ? (int)(row % n_pad) : 0;
    float acc = 0.f;
    if (valid_row && i < n) {
        const long off = (bh * (long)n + i) * DV + 8 * part;
        bf16x8 a = gload_bf16x8(o + off);
        bf16x8 b = gload_bf16x8(dout + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (valid_row && part == 0) {
        lse2[row] = i < n ? lse[bh * (long)n + i] * kLog2e : INFINITY;
        Dw[row] = acc;
    }
}

// ---------------------------------------------------------------- dK / dV

template <int D, int DV>
struct DkdvCfg {
    static constexpr int BN = 128;           // keys per workgroup, 32 per wave
    static constexpr int BM = 64;            // queries per step
};

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ Dw, bf16* __restrict__ dk, bf16* __restrict__ dvo, int n, int m,
    int n_pad, float scale, float c2) {
    using C = DkdvCfg<D, DV>;
    constexpr int BM = C::BM;
    // One LDS variable per buffer: the compiler can then tell that reads
    // of one buffer do not alias the asynchronous fills of the other, and
    // does not make them wait for those fills.
    __shared__ __align__(1024) bf16 sQ0[BM * D];
    __shared__ __align__(1024) bf16 sQ1[BM * D];
    __shared__ __align__(1024) bf16 sO0[BM * DV];
    __shared__ __align__(1024) bf16 sO1[BM * DV];
    __shared__ __align__(256) float sL0[BM];
    __shared__ __align__(256) float sL1[BM];
    __shared__ __align__(256) float sD0[BM];
    __shared__ __align__(256) float sD1[BM];
    auto pick = [](auto b_, auto* x0, auto* x1) __attribute__((always_inline)) {
        if constexpr (decltype(b_)::value == 0) return x0;
        else return x1;
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const long bh = blockIdx.x;
    const int j0 = blockIdx.y * C::BN;
    const int kw0 = j0 + 32 * wave;
    const int myk = kw0 + li;

    const bf16* qh = q + bh * (long)n * D;
    const bf16* kh = k + bh * (long)m * D;
    const bf16* vh = v + bh * (long)m * DV;
    const bf16* oh = dout + bh * (long)n * DV;
    const float* lh = lse2 + bh * (long)n_pad;
    const float* dh = Dw + bh * (long)n_pad;

    // This lane's key row: B operand of S = Q K^T and of dP = dO V^T.
    bf16x8 kreg[D / 16], vreg[DV / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
        kreg[kc] = myk < m ? gload_bf16x8(kh + (long)myk * D + 16 * kc + 8 * g) : bf16x8{};
#pragma unroll
    for (int kc = 0; kc < DV / 16; ++kc)
        vreg[kc] = myk < m ? gload_bf16x8(vh + (long)myk * DV + 16 * kc + 8 * g) : bf16x8{};

    TileOffsets<D> toQ;
    toQ.init(lane);
    TileOffsets<DV> toO;
    toO.init(lane);

    const int i_begin = CAUSAL ? (j0 / BM) * BM : 0;
    const int i_end = (n + BM - 1) / BM * BM;
    const int nsteps = (i_end - i_begin) / BM;

    // Stage query tile i0 into a buffer: Q and dO rows (rows past n come
    // back as zeros; their LSE2 is +inf, so P = 0 and they contribute
    // nothing), and the per-row LSE2 and D.
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(qh, (uint32_t)n * D * 2);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(oh, (uint32_t)n * DV * 2);
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(lh, (uint32_t)n_pad * 4);
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(dh, (uint32_t)n_pad * 4);
    TileLoader<D, BM, 4> ldQ;
    ldQ.init(wave, lane);
    TileLoader<DV, BM, 4> ldO;
    ldO.init(wave, lane);
    auto stage = [&](auto buf_, int i0) __attribute__((always_inline)) {
        tile_fill<D, BM, 4>(ldQ, pick(buf_, sQ0, sQ1), rQ, i0, wave);
        tile_fill<DV, BM, 4>(ldO, pick(buf_, sO0, sO1), rO, i0, wave);
        if (wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (ATTN_LDS void*)pick(buf_, sL0, sL1), 4,
                                                     4 * lane, 4 * i0, 0, 0);
        else if (wave == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (ATTN_LDS void*)pick(buf_, sD0, sD1), 4,
                                                     4 * lane, 4 * i0, 0, 0);
    };

    f32x16 accK[D / 32], accV[DV / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) accK[t] = zero16();
#pragma unroll
    for (int t = 0; t < DV / 32; ++t) accV[t] = zero16();

    // One query tile.  The step is a fixed sequence of NA + NC products,
    // issued one per slot in this order:
    //   A ops (per query half t): S[t] += Q_t K^T (D/16), dP[t] += dO_t V^T (DV/16)
    //   C ops (per t, c):         dV += P^T dO (DV/32), dK += dS^T Q (D/32)
    // Each product's LDS operand is fetched PD slots ahead, and the softmax
    // of one half is spread over the slots of the other half's products, so
    // that the matrix cores, the LDS and the vector ALUs work at the same
    // time.  Slots are fenced with sched_barrier so the compiler keeps this
    // order.  MASKED steps apply the causal mask (tiles on the diagonal).
    auto compute = [&](auto buf_, auto masked_, int i0) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_)::value;
        const bf16* Qs = pick(buf_, sQ0, sQ1);
        const bf16* Os = pick(buf_, sO0, sO1);
        const float* Ls = pick(buf_, sL0, sL1);
        const float* Dsm = pick(buf_, sD0, sD1);

        constexpr int KA = D / 16, KB = DV / 16;
        constexpr int NAT = KA + KB, NA = 2 * NAT;
        constexpr int NCX = DV / 32 + D / 32;
        constexpr int NCT = 2 * NCX, NC = 2 * NCT;
        constexpr int NOPS = NA + NC;
        constexpr int PD = 4;

        auto load_op = [&](auto oc_) __attribute__((always_inline)) -> bf16x8 {
            constexpr int o = decltype(oc_)::value;
            if constexpr (o < NA) {
                constexpr int t = o / NAT, r = a_order<KA, KB>(o % NAT);
                if constexpr (r < KA) return tile_read8_at<D>(Qs, toQ, 32 * t, r);
                else return tile_read8_at<DV>(Os, toO, 32 * t, r - KA);
            } else {
                constexpr int oc = o - NA;
                constexpr int t = oc / NCT, rc = oc % NCT;
                constexpr int c = rc / NCX, x = rc % NCX;
                if constexpr (x < DV / 32) return tile_read_tr_at<DV>(Os, toO, 32 * t + 16 * c, x);
                else return tile_read_tr_at<D>(Qs, toQ, 32 * t + 16 * c, x - DV / 32);
            }
        };

        f32x16 S[2], dP[2];
        bf16x8 Pb[2][2], dSb[2][2];
        f32x4 l4[4], d4[4];
        float p[16], ds[16];

        // key > query  <=>  32t + 8vq + r < myk - i0 - 4g
        const int mask_lim = myk - i0 - 4 * g;
        auto load_stats = [&](auto t_, auto vq_) __attribute__((always_inline)) {
            constexpr int t = decltype(t_)::value, vq = decltype(vq_)::value;
            l4[vq] = *reinterpret_cast<const f32x4*>(Ls + 32 * t + 8 * vq + 4 * g);
            d4[vq] = *reinterpret_cast<const f32x4*>(Dsm + 32 * t + 8 * vq + 4 * g);
        };
        // One accumulator slot E of half T: P = exp2(S*scale*log2e - LSE2),
        // dS = P (dP - D); after slots 7 and 15 the eight values are rounded
        // to bf16 as one operand.
        auto softmax_elem = [&](auto t_, auto e_) __attribute__((always_inline)) {
            constexpr int t = decltype(t_)::value, e = decltype(e_)::value;
            constexpr int vq = e >> 2, r = e & 3;
            float pv = fast_exp2(__builtin_fmaf(S[t][e], c2, -l4[vq][r]));
            if constexpr (MASKED) pv = (32 * t + 8 * vq + r < mask_lim) ? 0.f : pv;
            p[e] = pv;
            ds[e] = pv * (dP[t][e] - d4[vq][r]);
            if constexpr ((e & 7) == 7) {
                constexpr int c = e >> 3, b = 8 * c;
                Pb[t][c] = pack8(p[b], p[b + 1], p[b + 2], p[b + 3], p[b + 4], p[b + 5], p[b + 6], p[b + 7]);
                dSb[t][c] = pack8(ds[b], ds[b + 1], ds[b + 2], ds[b + 3], ds[b + 4], ds[b + 5],
                                  ds[b + 6], ds[b + 7]);
            }
        };

        // The softmax of each half is spread one or two accumulator slots per
        // product over a window of slots, so that its exponentials and
        // conversions overlap the matrix products instead of stalling them:
        // half 0 over the A ops of half 1, half 1 over the C ops of half 0
        // (finishing each bf16 operand before the first product that reads it).
        constexpr int W0[2] = {NAT + 2, NA + 2};
        constexpr int W1[2] = {NA, NA + NCT + NCX - 1};
        static_assert(W1[0] > W0[0] && W1[1] > W0[1], "softmax windows");
        static_assert(W0[1] + (7 * (W1[1] - W0[1])) / 16 < NA + NCT, "half 1 low operand in time");

        bf16x8 fr[PD];
        static_for<PD>([&](auto o_) { fr[decltype(o_)::value] = load_op(o_); });
        __builtin_amdgcn_sched_barrier(0);

        static_for<NOPS>([&](auto o_) {
            constexpr int o = decltype(o_)::value;
            const bf16x8 cur = fr[o % PD];
            if constexpr (o + PD < NOPS)
                fr[o % PD] = load_op(std::integral_constant<int, o + PD>{});
            if constexpr (o < NA) {
                constexpr int t = o / NAT, r = a_order<KA, KB>(o % NAT);
                if constexpr (o % NAT == 0) {
                    S[t] = zero16();
                    dP[t] = zero16();
                }
                if constexpr (r < KA) S[t] = mfma32(cur, kreg[r], S[t]);
                else dP[t] = mfma32(cur, vreg[r - KA], dP[t]);
            } else {
                constexpr int oc = o - NA;
                constexpr int t = oc / NCT, rc = oc % NCT;
                constexpr int c = rc / NCX, x = rc % NCX;
                if constexpr (x < DV / 32) accV[x] = mfma32(Pb[t][c], cur, accV[x]);
                else accK[x - DV / 32] = mfma32(dSb[t][c], cur, accK[x - DV / 32]);
            }
            static_for<2>([&](auto t_) {
                constexpr int t = decltype(t_)::value;
                constexpr int L = W1[t] - W0[t];
                // statistics for row group vq one slot before its first element
                static_for<4>([&](auto vq_) {
                    constexpr int vq = decltype(vq_)::value;
                    if constexpr (W0[t] + (4 * vq * L) / 16 - 1 == o) load_stats(t_, vq_);
                });
                static_for<16>([&](auto e_) {
                    constexpr int e = decltype(e_)::value;
                    if constexpr (W0[t] + (e * L) / 16 == o) softmax_elem(t_, e_);
                });
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

    int s = 0;
    if constexpr (CAUSAL) {
        // Query tiles that overlap keys j0..j0+BN-1 straddle the diagonal;
        // with BN = 2 BM these are the first two, buffers 0 and 1.
        static_assert(C::BN == 2 * BM, "two masked steps per key block");
        if (s < nsteps) do_step(B0{}, MaskOn{}, s++);
        if (s < nsteps) do_step(B1{}, MaskOn{}, s++);
    }
    for (; s + 1 < nsteps; s += 2) {
        do_step(B0{}, MaskOff{}, s);
        do_step(B1{}, MaskOff{}, s + 1);
    }
    if (s < nsteps) do_step(B0{}, MaskOff{}, s);

    // Accumulator slot vv of tile nt holds key kw0 + 8*(vv>>2) + 4g + (vv&3),
    // column 32*nt + li.
    bf16* dkh = dk + bh * (long)m * D;
    bf16* dvh = dvo + bh * (long)m * DV;
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
        const int key = kw0 + 8 * (vv >> 2) + 4 * g + (vv & 3);
        if (key < m) {
#pragma unroll
            for (int nt = 0; nt < D / 32; ++nt)
                dkh[(long)key * D + 32 * nt + li] = (bf16)(accK[nt][vv] * scale);
#pragma unroll
            for (int nt = 0; nt < DV / 32; ++nt)
                dvh[(long)key * DV + 32 * nt + li] = (bf16)accV[nt][vv];
        }
    }
}

template <int DV>
void launch_pre(const Problem& p, const void* o, const void* dout, const float* lse,
                const Workspace& w, hipStream_t s) {
    constexpr int RPB = 256 / (DV / 8);
    const long total = p.heads() * (long)w.n_pad;
    const unsigned blocks = (unsigned)((total + RPB - 1) / RPB);
    bwd_preprocess_kernel<DV><<<blocks, 256, 0, s>>>((const bf16*)o, (const bf16*)dout, lse,
                                                     w.lse2, w.D, p.n, w.n_pad, total);
}

template <int D, int DV>
void launch_dkdv(const Problem& p, const void* q, const void* k, const void* v,
                 const void* dout, const Workspace& w, void* dk, void* dv, hipStream_t s) {
    using C = DkdvCfg<D, DV>;
    dim3 grid((unsigned)p.heads(), (unsigned)((p.m + C::BN - 1) / C::BN));
    const float c2 = p.scale * kLog2e;
    if (p.causal)
        bwd_dkdv_kernel<D, DV, true><<<grid, 256, 0, s>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, w.lse2, w.D,
            (bf16*)dk, (bf16*)dv, p.n, p.m, w.n_pad, p.scale, c2);
    else
        bwd_dkdv_kernel<D, DV, false><<<grid, 256, 0, s>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, w.lse2, w.D,
            (bf16*)dk, (bf16*)dv, p.n, p.m, w.n_pad, p.scale, c2);
}

}  // namespace

bool launch_bwd_preprocess_bf16(const Problem& p, const void* o, const void* dout,
                                const float* lse, const Workspace& w, hipStream_t s) {
    if (p.dv == 64) launch_pre<64>(p, o, dout, lse, w, s);
    else if (p.dv == 128) launch_pre<128>(p, o, dout, lse, w, s);
    else return false;
    return true;
}

bool launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                          const void* dout, const Workspace& w, void* dk, void* dv,
                          hipStream_t s) {
    if (p.d == 64 && p.dv == 64) launch_dkdv<64, 64>(p, q, k, v, dout, w, dk, dv, s);
    else if (p.d == 128 && p.dv == 128) launch_dkdv<128, 128>(p, q, k, v, dout, w, dk, dv, s);
    else if (p.d == 128 && p.dv == 64) launch_dkdv<128, 64>(p, q, k, v, dout, w, dk, dv, s);
    else return false;
    return true;
}

}  // namespace attn

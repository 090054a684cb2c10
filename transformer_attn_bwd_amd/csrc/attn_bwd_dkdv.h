// dK/dV kernel of backward attention on 16-bit MFMA (bf16 or f16 inputs,
// float32 accumulation), shared by three objects: attn_bwd_mfma.hip builds
// it without dQ work, attn_bwd_dkdv_dqa.hip with the fused dQ contribution
// below (DQA), attn_bwd_dkdv_dss.hip writing its dS to the workspace for
// the dQ-from-dS pass (DSS).
//
// One workgroup per 256 keys of a head (64 per wave) walks the query tiles,
// recomputes S = Q K^T and P, and accumulates dV += P^T dO and dK += dS^T Q
// in registers (eulerpad "Attention backward" P2, P6).  The lane owns a key:
// the accumulator layout of S (rows = queries, columns = keys) is exactly
// the A-operand layout P^T and dS^T need (rows = keys, k = queries), so P
// and dS never leave registers; the partners dO and Q are read with
// transposing LDS reads in the matching row-of-C order.  The causal mask
// (S_ij = -inf for j > i, i.e. P_ij = 0, eulerpad P8) is applied only in
// tiles that straddle the diagonal; tiles entirely above it are never
// visited.
//
// Fused dQ (DQA = true, for workgroups whose first key is at or past
// dqa_from): dQ_i = sum_j dS_ij K_j (eulerpad P5; scale applied later) over
// this workgroup's 256 keys is added to a float32 accumulator in global
// memory with atomics, so that the separate dQ pass only covers the keys
// before dqa_from.  dS leaves the registers once per step: each wave writes
// its 64 x 32 tile of dS (keys x queries) to LDS, and after the step's
// barrier wave w multiplies the whole 256 x 32 tile by a block of K,
// dQ[32 queries][32 columns] += dS[q][keys] K[keys][cols], during the S
// products of the next step, parks the 16 float32 values per lane in LDS,
// and sends them to the accumulator with global atomic adds at the start
// of the step after that (so that the wait closing a step, which covers
// the next tile's loads, never waits on atomics just issued).
#pragma once

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

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
// half of the step, x: 32-column block).  With the fused dQ, the step
// starts with the previous step's dQ product,
//   dQ  4NX  MFMAs  dQ[32 q][block] += dS_prev[q][keys of chunk t] K[keys][block]
// while none of the step's softmax values are live, and slot J_QST parks
// the finished product in LDS.
// Operand fragments read from LDS:
//   f <  KA               Q rows, chunk f              (first used by j = 2f)
//   f < 3KA               K rows of tile kt, chunk r   (j = 2r + kt)
//   f < 3KA + KB          dO rows, chunk r             (j = 2KA + 2r)
//   f < 3KA + KB + 2NXV   dO^T half c, block x         (dV, first j of (c, x))
//   f < F_QS              Q^T half c, block x          (dK, first j of (c, x))
//   f < F_QK              dS_prev chunk t (fused dQ, read before the slots)
//   f < NF_QA             K^T chunk t, this wave's block (fused dQ)
template <int D, int DV>
struct DkdvSched {
    static constexpr int KA = D / 16, KB = DV / 16, NX = D / 32, NXV = DV / 32;
    static constexpr int J_DP = 2 * KA, J_DV = J_DP + 2 * KB, J_DK = J_DV + 4 * NXV;
    static constexpr int NJ = J_DK + 4 * NX;
    static constexpr int F_K = KA, F_DO = 3 * KA, F_DOT = F_DO + KB, F_QT = F_DOT + 2 * NXV;
    static constexpr int NF = F_QT + 2 * NX;
    static constexpr int NQ = 4 * NX;        // fused dQ MFMAs per step (= S slots, 2 KA)
    static constexpr int J_QST = 4;          // slot that parks the finished product
    static constexpr int F_QS = NF, F_QK = NF + NQ, NF_QA = NF + 2 * NQ;
    static constexpr int first_use(int f) {
        if (f < F_K) return 2 * f;
        if (f < F_DO) return 2 * ((f - F_K) % KA) + (f - F_K) / KA;
        if (f < F_DOT) return J_DP + 2 * (f - F_DO);
        if (f < F_QT) return J_DV + 2 * (f - F_DOT);
        return J_DK + 2 * (f - F_QT);
    }
    static constexpr int LAQ = 2;            // fused-dQ fragments are read this many MFMAs ahead
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
    // statistics of row group vq (accumulator slots 4vq..4vq+3): LSE2 is
    // read two slots before the first element that needs it, -D (the
    // starting value of the dP accumulators) four slots before dP
    static constexpr int first_elem_of_vq(int vq) { return 16 * (vq / 2) + 4 * (vq % 2); }
    static constexpr int l_slot(int vq) { return p_slot(first_elem_of_vq(vq)) - 2; }
    static constexpr int d_slot(int vq) { return J_DP - 4 + vq; }
};

// The dS tile of the fused dQ: 256 keys x 32 queries, 16-bit, one 64-byte
// row per key.  The 8-byte column groups of row r sit at group g ^ sw(r),
// sw(r) = (r >> 2) & 7: each wave's writes (32 keys, one column group)
// and the transposing reads (4 keys x 8 groups per 32 lanes) then both touch
// every bank once.
constexpr int kDsCols = 32;

// dS stores per wave and step in the stored-dS kernel: four 8-value packs,
// each as two 8-byte stores; also the vmcnt field of the step's closing
// s_waitcnt (expcnt and lgkmcnt fields zero).
constexpr int kDssStores = 8;

// The lane index, computed where it is needed: the asm cannot be moved out
// of a loop, so no register holds the index (or values derived from it)
// through one.
__device__ __forceinline__ int lane_id_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
__device__ __forceinline__ int ds_tile_off(int r, int cgrp) {
    return r * kDsCols + 4 * (cgrp ^ ((r >> 2) & 7));
}

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
template <typename T, int D, int DV, bool CAUSAL, bool DQA, bool DSS>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ Dw, T* __restrict__ dk, T* __restrict__ dvo,
    float* __restrict__ dqacc, int dqa_from, int n, int m, int dg, int dvg, int n_pad,
    float scale, float c2, SeqInfo si, DsTiles dst) {
    using C = DkdvCfg<D, DV>;
    using SC = DkdvSched<D, DV>;
    // the 128/128 kernel without the fused dQ forms P and dS slots before
    // the products that read them (checked in the assembly at build time)
    constexpr bool kOperandWait = DQA || D != 128 || DV != 128;
    static_assert(!(DQA && DSS), "one dQ mode per instantiation");
    constexpr int BM = C::BM, NW = C::NW, LA = C::LA;
    // One LDS variable per buffer: the compiler can then tell that reads
    // of one buffer do not alias the asynchronous fills of the other, and
    // does not make them wait for those fills.  The streaming tiles (4 or
    // 8 KB, aligned to their size) are aligned more strictly than the K tile
    // so that they are placed first, below 64 KB: their reads then take the
    // buffer's address as the instruction's 16-bit immediate offset instead
    // of an add per read.
    __shared__ __align__(BM * D * sizeof(T)) T sQ0[BM * D];
    __shared__ __align__(BM * D * sizeof(T)) T sQ1[BM * D];
    __shared__ __align__(BM * DV * sizeof(T)) T sO0[BM * DV];
    __shared__ __align__(BM * DV * sizeof(T)) T sO1[BM * DV];
    __shared__ __align__(1024) T sK[C::BN * D];
    __shared__ __align__(256) float sL0[64];
    __shared__ __align__(256) float sL1[64];
    __shared__ __align__(256) float sD0[64];
    __shared__ __align__(256) float sD1[64];
    // dS tiles of the fused dQ, one per step parity (unused without it)
    __shared__ __align__(1024) T sS0[DQA ? C::BN * kDsCols : 1];
    __shared__ __align__(1024) T sS1[DQA ? C::BN * kDsCols : 1];
    // the finished dQ product of each wave between its MFMAs and its atomics
    __shared__ __align__(1024) float sQacc[DQA ? NW * 64 * 16 : 1];
    auto pick = [](auto b_, auto* x0, auto* x1) __attribute__((always_inline)) {
        if constexpr (decltype(b_)::value == 0) return x0;
        else return x1;
    };

    // the wave index is uniform: computed once into a scalar register, so
    // that the LDS addresses of the tile fills (M0) need no per-load
    // vector-to-scalar move
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const TileOrder to = tile_order((int)gridDim.x, (int)gridDim.y);
    const long bh = to.head;
    const int j0 = to.rank * C::BN;
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

    // Fused dQ.  Wave w computes the 32-column block xq of dQ over the keys
    // kq0 .. kq0 + 64 NX - 1 of the workgroup (all 256 for D = 128; half of
    // them for D = 64, where two waves share a block and both add).  The
    // last key block may reach past mb: dS of those keys is written as zero
    // (their K rows are zero, but P there is not bounded, so dS could be
    // infinite).  The kernel uses every register at D = DV = 128, so the
    // per-lane offsets of the fused dQ are recomputed where they are used,
    // from a copy of the lane index the compiler cannot hoist (asm barrier),
    // instead of being kept through the loop.
    const bool dqa_on = DQA && j0 >= dqa_from;
    const bool ragged = j0 + C::BN > mb;
    // Stored dS (DSS): this head's tiles, and this wave's 64 key rows of
    // them (32768 bytes per 64 rows of 256 queries).
    const __amdgpu_buffer_rsrc_t rds =
        make_rsrc(DSS ? reinterpret_cast<const T*>(dst.p) + bh * dst.head_elems : q,
                  DSS ? (uint32_t)(dst.head_elems * 2) : 0u);
    const int kblk = to.rank;
    constexpr int NXQ = D / 32, WPB = NW / NXQ;
    const int xq = wave % NXQ, kq0 = (wave / NXQ) * (C::BN / WPB);
    auto opaque_lane = []() __attribute__((always_inline)) { return lane_id_here(); };
    // transposing reads of a 16-key chunk of parity p of the dS tile
    // (relative to the chunk's first row: the swizzle of row 16t + r depends
    // on t only through t's parity), piece h
    auto ds_rd_off = [](int l, int p, int h) __attribute__((always_inline)) {
        const int gg = l >> 5, j = l & 15, blk = l >> 4;
        return ds_tile_off(16 * p + 4 * gg + (j >> 2) + 8 * h, 4 * (blk & 1) + (j & 3)) -
               16 * p * kDsCols;
    };
    // transposing reads of K's column block xq, piece h (the layout of
    // TileOffsets::tr)
    auto kq_tr_off = [&](int l, int h) __attribute__((always_inline)) {
        const int gg = l >> 5, j = l & 15, blk = l >> 4;
        const int r = 4 * gg + (j >> 2) + 8 * h;
        const int col = 32 * xq + 16 * (blk & 1) + 4 * (j & 3);
        return SwzTile<D>::off(r, col >> 3) + (col & 7);
    };
    f32x16 accQ;
    // dQ rows i0 .. i0 + 31 of a finished product go out as 16 atomic adds
    // per lane: slot e is row 8(e>>2) + 4g + (e&3), column 32 xq + li.
    auto dq_atomics = [&](const f32x16& a, int i0) __attribute__((always_inline)) {
        const int l = opaque_lane();
        float* p0 = dqacc + (bh * (long)n_pad + i0 + 4 * (l >> 5)) * D + 32 * xq + (l & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            __hip_atomic_fetch_add(p0 + (8 * (e >> 2) + (e & 3)) * D, a[e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    };
    // The finished product waits in this lane's 16 floats of sQacc.
    auto park_ptr = [&]() __attribute__((always_inline)) {
        return sQacc + (wave * 64 + opaque_lane()) * 16;
    };
    auto dq_park = [&]() __attribute__((always_inline)) {
        float* pk = park_ptr();
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
            *reinterpret_cast<f32x4*>(pk + 4 * v4) =
                f32x4{accQ[4 * v4], accQ[4 * v4 + 1], accQ[4 * v4 + 2], accQ[4 * v4 + 3]};
    };
    auto dq_atomics_parked = [&](int i0) __attribute__((always_inline)) {
        const float* pk = park_ptr();
        f32x16 a;
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(pk + 4 * v4);
#pragma unroll
            for (int r = 0; r < 4; ++r) a[4 * v4 + r] = x[r];
        }
        dq_atomics(a, i0);
    };

    // One query tile: the SC schedule, one MFMA per slot (two in the dK
    // slots with the fused dQ), fenced with sched_barrier so that the
    // operand reads (LA slots ahead), the matrix products and the softmax
    // work interleave as written.  MASKED steps apply the causal mask.
    auto compute = [&](auto buf_, auto masked_, int i0) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_)::value;
        constexpr int NF = DQA ? SC::NF_QA : SC::NF;
        const T* Qs = pick(buf_, sQ0, sQ1);
        const T* Os = pick(buf_, sO0, sO1);
        const float* Ls = pick(buf_, sL0, sL1);
        const float* Ds = pick(buf_, sD0, sD1);
        // this step's dS tile and the previous step's
        T* Scur = pick(buf_, sS0, sS1);
        const T* Sprev = pick(std::integral_constant<int, decltype(buf_)::value ^ 1>{}, sS0, sS1);
        // offsets of the fused-dQ reads, set at the start of the dQ phase:
        // dS chunks of parity 0 and 1, then K's block xq
        int qoff[3][2];

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
            } else if constexpr (f < SC::F_QS) {
                constexpr int c = (f - SC::F_QT) / SC::NX, x = (f - SC::F_QT) % SC::NX;
                return tile_read_tr_at<D>(Qs, toQ, 16 * c, x);
            } else if constexpr (f < SC::F_QK) {
                // dS_prev rows kq0 + 16t .. +15 (keys), column = query of the lane
                constexpr int t = f - SC::F_QS;
                const T* b = Sprev + (kq0 + 16 * t) * kDsCols;
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(b + qoff[t & 1][0]));
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(b + qoff[t & 1][1]));
                i16x4 both[2] = {lo, hi};
                return *reinterpret_cast<vec8<T>*>(both);
            } else {
                // K rows kq0 + 16t .. +15, column 32 xq + (lane & 31)
                constexpr int t = f - SC::F_QK;
                const T* b = sK + (kq0 + 16 * t) * D;
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(b + qoff[2][0]));
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(b + qoff[2][1]));
                i16x4 both[2] = {lo, hi};
                return *reinterpret_cast<vec8<T>*>(both);
            }
        };

        f32x16 S[2], dP[2];          // S is overwritten by P
        vec8<T> Pb[2][2], dSb[2][2];
        f32x4 l4[4];
        f32x16 nD;   // -D of the accumulator rows: slot 4vq + r is row 8vq + 4g + r
        vec8<T> fr[NF];

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
            constexpr int kt = SC::elem_kt(i), e = SC::elem_e(i);
            dP[kt][e] = S[kt][e] * dP[kt][e];   // dP already holds dO V^T - D
            if constexpr (i % 8 == 7) {
                constexpr int c = SC::elem_c(i), b = 8 * c;
                dSb[kt][c] = pack8<T>(dP[kt][b], dP[kt][b + 1], dP[kt][b + 2], dP[kt][b + 3],
                                   dP[kt][b + 4], dP[kt][b + 5], dP[kt][b + 6], dP[kt][b + 7]);
            }
        };
        // dS pack (kt, c) of this lane's key into this step's tile: two
        // 8-byte pieces (queries 16c + 4g .. +3 and 16c + 8 + 4g .. +3)
        auto ds_store = [&](auto p_) __attribute__((always_inline)) {
            constexpr int p = decltype(p_)::value, kt = p % 2, c = p / 2;
            const int l = opaque_lane();
            vec8<T> w = dSb[kt][c];
            if (ragged) w = kw0 + 32 * kt + (l & 31) < mb ? w : vec8<T>{};
            T* b = Scur + (C::KW * wave + 32 * kt) * kDsCols;
            const int r = l & 31, gg = l >> 5;
            *reinterpret_cast<vec4<T>*>(b + ds_tile_off(r, 4 * c + gg)) = vec4<T>{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<vec4<T>*>(b + ds_tile_off(r, 4 * c + 2 + gg)) = vec4<T>{w[4], w[5], w[6], w[7]};
        };

        // Stored dS: pack (kt, c) of this lane's key goes to key row
        // 64 wave + 32 kt + (lane & 31) of the step's [256 keys][32 queries]
        // block of tile (i0 / 256, kblk), columns 16c + 4g .. +3 and
        // 16c + 8 + 4g .. +3 (two 8-byte stores).  The block is contiguous,
        // so the four stores of a key tile fill whole 128-byte lines
        // together.
        auto ds_gstore = [&](auto p_) __attribute__((always_inline)) {
            constexpr int p = decltype(p_)::value, kt = p % 2, c = p / 2;
            const int l = opaque_lane();
            vec8<T> w = dSb[kt][c];
            if (ragged) w = kw0 + 32 * kt + (l & 31) < mb ? w : vec8<T>{};
            const u32x4 bits = __builtin_bit_cast(u32x4, w);
            const int b = i0 / kDsTile;
            const long tile = dst.tri ? (long)b * (b + 1) / 2 + kblk : (long)b * dst.mblk + kblk;
            const uint32_t so =
                (uint32_t)((tile * kDsTile * kDsTile + (i0 % kDsTile) * kDsTile) * 2) +
                (uint32_t)(64 * BM * 2 * wave);
            const uint32_t vo = (uint32_t)((l & 31) * (BM * 2) + (l >> 5) * 8 + 32 * c +
                                           32 * BM * 2 * kt);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{bits[0], bits[1]}, rds, vo, so, 0);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{bits[2], bits[3]}, rds, vo + 16, so, 0);
        };

        // Fused dQ first: the previous step's product, before this step's
        // products, while the softmax values of the step are not yet live.
        if constexpr (DQA) {
            if (dqa_on) {
                const int l = opaque_lane();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    qoff[0][h] = ds_rd_off(l, 0, h);
                    qoff[1][h] = ds_rd_off(l, 1, h);
                    qoff[2][h] = kq_tr_off(l, h);
                }
                static_for<SC::NQ + SC::LAQ>([&](auto u_) {
                    constexpr int u = decltype(u_)::value;
                    if constexpr (u < SC::NQ) {
                        fr[SC::F_QS + u] = load_frag(std::integral_constant<int, SC::F_QS + u>{});
                        fr[SC::F_QK + u] = load_frag(std::integral_constant<int, SC::F_QK + u>{});
                    }
                    if constexpr (u >= SC::LAQ) {
                        constexpr int t = u - SC::LAQ;
                        accQ = mfma32(fr[SC::F_QS + t], fr[SC::F_QK + t], t == 0 ? zero16() : accQ);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        }

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
                if constexpr (SC::d_slot(vq) == j) {
                    const f32x4 t4 = *reinterpret_cast<const f32x4*>(Ds + 8 * vq + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) nD[4 * vq + r] = t4[r];
                }
            });
            // the product of this slot
            constexpr int kt = j % 2;
            if constexpr (DQA && j == SC::J_QST) {
                if (dqa_on) dq_park();
            }
            if constexpr (j < SC::J_DP) {
                constexpr int r = j / 2;
                if constexpr (r == 0) S[kt] = zero16();
                S[kt] = mfma32(fr[r], fr[SC::F_K + kt * SC::KA + r], S[kt]);
            } else if constexpr (j < SC::J_DV) {
                constexpr int r = (j - SC::J_DP) / 2;
                dP[kt] = mfma32(fr[SC::F_DO + r], vreg[kt][r], r == 0 ? nD : dP[kt]);
            } else if constexpr (j < SC::J_DK) {
                constexpr int cx = (j - SC::J_DV) / 2, c = cx / SC::NXV, x = cx % SC::NXV;
                mfma32_agpr<kOperandWait>(fr[SC::F_DOT + cx], Pb[kt][c], accV[kt][x]);
            } else {
                constexpr int cx = (j - SC::J_DK) / 2, c = cx / SC::NX, x = cx % SC::NX;
                mfma32_agpr<kOperandWait>(fr[SC::F_QT + cx], dSb[kt][c], accK[kt][x]);
                if constexpr (DQA) {
                    constexpr int t = j - SC::J_DK;
                    if constexpr (t < 4) {
                        if (dqa_on) ds_store(std::integral_constant<int, t>{});
                    }
                }
                if constexpr (DSS) {
                    constexpr int t = j - SC::J_DK;
                    if constexpr (t < 4) ds_gstore(std::integral_constant<int, t>{});
                }
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

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using MaskOn = std::integral_constant<bool, true>;
    using MaskOff = std::integral_constant<bool, false>;

    // The step loop.  With the fused dQ, step s computes the dQ product of
    // step s - 1 (whose dS tile the barrier closing step s - 1 made
    // visible) and, at its start, after requesting the next query tile,
    // sends the product of step s - 2.
    {
        auto do_step = [&](auto buf_, auto masked_, int s) __attribute__((always_inline)) {
            constexpr int buf = decltype(buf_)::value;
            const int i0 = i_begin + s * BM;
            if (s + 1 < nsteps) stage(std::integral_constant<int, buf ^ 1>{}, i0 + BM);
            if constexpr (DQA) {
                if (dqa_on && s >= 2) dq_atomics_parked(i0 - 2 * BM);
            }
            compute(buf_, masked_, i0);
            if constexpr (DSS) {
                // The next tile's loads were issued before this step's eight
                // dS stores, and vector memory operations count down in the
                // order they were issued: waiting until at most eight
                // remain waits for the loads and leaves the stores in
                // flight (lgkmcnt(0): this step's LDS accesses are done).
                __builtin_amdgcn_s_waitcnt(kDssStores);
            } else {
                __builtin_amdgcn_s_waitcnt(0);
            }
            __syncthreads();
        };

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

        if (DQA && dqa_on) {
            // the product of the second-to-last step is in accQ; the last
            // step's dS tile is complete (the loop ended on a barrier)
            if (nsteps >= 2) dq_atomics_parked(i_begin + (nsteps - 2) * BM);
            if (nsteps >= 1) {
                const T* Sl = ((nsteps - 1) & 1) ? sS1 : sS0;
                const int l = opaque_lane();
                accQ = zero16();
#pragma unroll
                for (int t = 0; t < SC::NQ; ++t) {
                    const T* bs = Sl + (kq0 + 16 * t) * kDsCols;
                    const T* bk = sK + (kq0 + 16 * t) * D;
                    i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(bs + ds_rd_off(l, t & 1, 0)));
                    i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(bs + ds_rd_off(l, t & 1, 1)));
                    i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(bk + kq_tr_off(l, 0)));
                    i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(bk + kq_tr_off(l, 1)));
                    i16x4 aa[2] = {a0, a1}, bb[2] = {b0, b1};
                    accQ = mfma32(*reinterpret_cast<vec8<T>*>(aa), *reinterpret_cast<vec8<T>*>(bb), accQ);
                }
                dq_atomics(accQ, i_begin + (nsteps - 1) * BM);
            }
            // other waves may still read the K tile, which the epilogue reuses
            __syncthreads();
        }
    }

    // wait states between the last MFMA writing an accumulator and the
    // reads below, and no read of an accumulator before them
    mfma_agpr_wait();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int x = 0; x < D / 32; ++x) mfma_agpr_fence(accK[kt][x]);
#pragma unroll
        for (int x = 0; x < DV / 32; ++x) mfma_agpr_fence(accV[kt][x]);
    }

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
    // negative).  Only a wave whose 64 keys reach past mb takes the
    // selecting copy of the epilogue.
    T* reg = sK + C::KW * wave * D;
    auto put_tile = [&](auto W_, auto RAGGED_, const f32x16 (&acc)[2][W_.value / 32], int wcols,
                        float mult, T* out, long stride) __attribute__((always_inline)) {
        constexpr int W = decltype(W_)::value;
        constexpr bool RAGGED = decltype(RAGGED_)::value;
        constexpr int SW = W < D ? W : D;      // slab width: what the region holds
        constexpr int CH = SW / 8;             // 16-byte chunks per slab row
        constexpr int RPI = 64 / CH;           // rows per store instruction
        // Stores go through a buffer resource ending after key row m - 1; a
        // chunk past the last key or past the row's wcols columns gets an
        // offset beyond that end, and the hardware drops it (no branch).
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, (uint32_t)(m * stride * 2));
        // lane's row and chunk in store i: row RPI i + lane / CH, chunk lane % CH
        const int srow = lane / CH, schunk = lane % CH;
        const uint32_t row_step = (uint32_t)(RPI * stride * 2);
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
                        for (int r = 0; r < 4; ++r) w4[r] = (T)(acc[kt][x][4 * vq + r] * mult);
                        if constexpr (RAGGED) {
                            u32x2 b = __builtin_bit_cast(u32x2, w4);
                            b = real ? b : u32x2{0u, 0u};
                            w4 = __builtin_bit_cast(vec4<T>, b);
                        }
                        const int chunk = 4 * xs + vq;
                        *reinterpret_cast<vec4<T>*>(
                            reg + row * SW + 8 * (chunk ^ (row & (CH - 1))) + 4 * g) = w4;
                    }
                }
            }
            // every row read first, then every store: one wait for the reads
            vec8<T> w8[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int row = RPI * i + srow;
                w8[i] = *reinterpret_cast<const vec8<T>*>(
                    reg + row * SW + 8 * (schunk ^ (row & (CH - 1))));
            }
            const int col = sl * SW + 8 * schunk;
            const uint32_t off0 = (uint32_t)(((long)(kw0 + srow) * stride + col) * 2);
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const uint32_t byte_off = col < wcols ? off0 + (uint32_t)i * row_step : 0xFFFFFFF0u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w8[i]), ro,
                                                       byte_off, 0, 0);
            }
        }
    };
    using Dc = std::integral_constant<int, D>;
    using DVc = std::integral_constant<int, DV>;
    if (kw0 + C::KW <= mb) {
        put_tile(Dc{}, std::false_type{}, accK, dg, scale, dk + hk.base, hk.stride);
        put_tile(DVc{}, std::false_type{}, accV, dvg, 1.f, dvo + hv.base, hv.stride);
    } else {
        put_tile(Dc{}, std::true_type{}, accK, dg, scale, dk + hk.base, hk.stride);
        put_tile(DVc{}, std::true_type{}, accV, dvg, 1.f, dvo + hv.base, hv.stride);
    }
}

template <typename T, int D, int DV, bool DQA, bool DSS = false>
void launch_dkdv(const Problem& p, const void* q, const void* k, const void* v,
                 const void* dout, const Workspace& w, void* dk, void* dv, float* dqacc,
                 int dqa_from, hipStream_t s) {
    using C = DkdvCfg<D, DV>;
    dim3 grid((unsigned)p.heads(), (unsigned)((p.m + C::BN - 1) / C::BN));
    const float c2 = p.scale * kLog2e;
    const SeqInfo si = seq_info(p);
    if (p.causal)
        bwd_dkdv_kernel<T, D, DV, true, DQA, DSS><<<grid, 256, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (const T*)dout, w.lse2, w.D,
            (T*)dk, (T*)dv, dqacc, dqa_from, p.n, p.m, p.d, p.dv, w.n_pad, p.scale, c2, si,
            w.ds);
    else
        bwd_dkdv_kernel<T, D, DV, false, DQA, DSS><<<grid, 256, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (const T*)dout, w.lse2, w.D,
            (T*)dk, (T*)dv, dqacc, dqa_from, p.n, p.m, p.d, p.dv, w.n_pad, p.scale, c2, si,
            w.ds);
}

}  // namespace
}  // namespace attn

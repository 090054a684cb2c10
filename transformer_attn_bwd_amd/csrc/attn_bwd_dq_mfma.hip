// dQ of backward attention on 16-bit MFMA (bf16 or f16 inputs, float32
// accumulation).
//
// For query row i, dQ_i = scale * sum_j dS_ij K_j with dS = P o (dP - D)
// and dP = dO V^T ("Attention Backpropagation: Step by step derivation",
// sections Gradient of S and Gradient of Q and K; mlgrind "Backward";
// eulerpad P5).  This pass recomputes S, P and dP per key tile instead of
// reading a stored P, and needs no atomics: each workgroup owns its query
// rows and walks the keys.
//
// Layout: one workgroup per 256 queries of a head, four waves, each wave
// owning two 32-query MFMA tiles.  The lane owns a query column of the
// transposed products
//     S^T = K Q^T,   dP^T = V dO^T,   dQ^T += K^T dS^T,
// so this lane's rows of Q and dO are register-resident B operands, and
// the accumulator layout of dS^T (rows = keys) is the B operand of the dQ
// product in row-of-C order (see attn_device.h).  Every 64-key tile of K
// and V is staged once in LDS and each fragment read from it feeds two
// MFMAs, one per query tile of the wave.  The dQ accumulators live in
// AGPRs.  The causal mask (S_ij = -inf for
// j > i, i.e. P_ij = 0, eulerpad P8) is applied only in key tiles that
// reach past the workgroup's first query.
//
// Given O and the forward's LSE, the pass also does the preprocess for its
// own rows (D = rowsum(dO o O), LSE in base 2) in its prologue and writes
// them to the workspace for the dK/dV kernel that follows, which saves the
// separate preprocess launch and its second read of dO.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D, int DV>
struct DqCfg {
    static constexpr int NW = 4;              // waves per workgroup
    static constexpr int BM = 2 * 32 * NW;    // queries per workgroup
    static constexpr int BN = 64;             // keys per step
    static constexpr int PD = 4;              // operand reads issued ahead
};

// With dqacc non-null the pass covers only the keys before key_limit (the
// rest reach dQ through the atomics of the fused dK/dV kernel) and writes
// its unscaled float32 sums to dqacc, [B*H][n_pad][D], every row of its
// tile below n_pad (padded rows as zeros); otherwise it covers every key
// and writes dQ = scale * sum in T.
template <typename T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, float* __restrict__ lse2, float* __restrict__ Dw,
    const T* __restrict__ o, const float* __restrict__ lse, T* __restrict__ dq,
    float* __restrict__ dqacc, int key_limit, int n, int m, int dg, int dvg, int n_pad,
    float scale, float c2, SeqInfo si) {
    using C = DqCfg<D, DV>;
    constexpr int BN = C::BN, PD = C::PD, NW = C::NW;
    // the d = 128 kernels form dS a fragment before the products that read
    // it (checked in the assembly at build time)
    constexpr bool kOperandWait = D != 128;
    // One LDS variable per buffer: the compiler can then tell that reads
    // of one buffer do not alias the asynchronous fills of the other, and
    // does not make them wait for those fills.
    __shared__ __align__(1024) T sK0[BN * D];
    __shared__ __align__(1024) T sK1[BN * D];
    __shared__ __align__(1024) T sV0[BN * DV];
    __shared__ __align__(1024) T sV1[BN * DV];
    // the epilogue's staging rows: 64 rows x 64 columns per wave
    __shared__ __align__(1024) T sE[NW * 64 * 64];
    auto Kbuf = [&](auto b_) __attribute__((always_inline)) -> T* {
        if constexpr (decltype(b_)::value == 0) return sK0;
        else return sK1;
    };
    auto Vbuf = [&](auto b_) __attribute__((always_inline)) -> T* {
        if constexpr (decltype(b_)::value == 0) return sV0;
        else return sV1;
    };

    // the wave index is uniform: computed once into a scalar register, so
    // that the LDS addresses of the tile fills (M0) need no per-load
    // vector-to-scalar move
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const TileOrder to = tile_order((int)gridDim.x, (int)gridDim.y);
    const long bh = to.head;
    const int qb = CAUSAL ? (int)gridDim.y - 1 - to.rank : to.rank;
    const int i0 = qb * C::BM;
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

    // Query tile t of this wave: rows i0 + (BM/2) t + 32 wave + (0..31).
    // Taking one tile from each half of the workgroup's rows gives every
    // wave the same share of the masked diagonal work.  Rows past nb load
    // zeros and LSE2 = +inf, so their P, dS and dQ vanish.
    //
    // Every load of the prologue (Q and dO rows, the O rows and LSE of the
    // preprocess or the workspace's LSE2 and -D, and the first K and V tile)
    // is issued before anything waits for one, so that their latencies
    // overlap instead of adding up.
    int myq[2];
    bool okq[2];
    vec8<T> qreg[2][D / 16], oreg[2][DV / 16];
    float l2[2], nD[2];   // LSE2 and -D of the row
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        myq[t] = i0 + (C::BM / 2) * t + 32 * wave + li;
        const bool ok = okq[t] = myq[t] < nb;
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc)
            qreg[t][kc] = (ok && 16 * kc + 8 * g < dg)
                              ? gload8(qh + (long)myq[t] * hq.stride + 16 * kc + 8 * g)
                              : vec8<T>{};
#pragma unroll
        for (int kc = 0; kc < DV / 16; ++kc)
            oreg[t][kc] = (ok && 16 * kc + 8 * g < dvg)
                              ? gload8(oh + (long)myq[t] * ho.stride + 16 * kc + 8 * g)
                              : vec8<T>{};
    }
    vec8<T> orow[2][DV / 16];
    float lraw[2];
    if (o != nullptr) {
        const HeadView hov = head_view(si, bh, n, dvg);
        const T* orow0 = o + hov.base;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int kc = 0; kc < DV / 16; ++kc)
                orow[t][kc] = (okq[t] && 16 * kc + 8 * g < dvg)
                                  ? gload8(orow0 + (long)myq[t] * hov.stride + 16 * kc + 8 * g)
                                  : vec8<T>{};
            lraw[t] = okq[t] ? lse[bh * (long)n + myq[t]] : -INFINITY;
        }
    } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            l2[t] = okq[t] ? lse2[bh * (long)n_pad + myq[t]] : INFINITY;
            nD[t] = okq[t] ? Dw[bh * (long)n_pad + myq[t]] : 0.f;   // the workspace holds -D
        }
    }

    int k_end = CAUSAL ? min(mb, i0 + C::BM + off) : mb;
    if (i0 >= nb) k_end = 0;
    k_end = min(k_end, key_limit);
    const int nsteps = (max(k_end, 0) + BN - 1) / BN;
    // Leading steps that need no mask: keys visible from the workgroup's
    // first query (causal) and inside the mb keys.  The rest are masked.
    int n_plain = min(nsteps, mb / BN);
    if (CAUSAL) n_plain = min(n_plain, max(i0 + off + 1, 0) / BN);

    // Key tiles go to LDS buffer s & 1 for step s, fetched one step ahead.
    // Rows past mb (last tile only) come back as zeros; masked steps zero
    // their P.
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(kh, (uint32_t)mb * hk.stride * 2);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(vh, (uint32_t)mb * hv.stride * 2);
    TileLoader<D, BN, NW> ldK;
    ldK.init(wave, lane, dg, hk.stride);
    TileLoader<DV, BN, NW> ldV;
    ldV.init(wave, lane, dvg, hv.stride);
    auto stage = [&](auto buf_, int k0) __attribute__((always_inline)) {
        tile_fill<D, BN, NW>(ldK, Kbuf(buf_), rK, k0, wave);
        tile_fill<DV, BN, NW>(ldV, Vbuf(buf_), rV, k0, wave);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    if (nsteps > 0) stage(B0{}, 0);

    if (o != nullptr) {
        // The preprocess for this workgroup's rows, in the arithmetic order
        // of bwd_preprocess_kernel, so that both give the same bits: each
        // 8-column chunk c summed in order, then the chunks pairwise at
        // distances 8, 4, 2, 1 (16 chunks; 4, 2, 1 for 8).  This lane holds
        // the chunks c = 2 kc + g, so the last step is the exchange with the
        // lane 32 away.  Rows past nb get D = 0 and LSE2 = +inf, rows that
        // saw no key (LSE = -inf) LSE2 = +inf.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float sc[DV / 16];
#pragma unroll
            for (int kc = 0; kc < DV / 16; ++kc) {
                const vec8<T> a = orow[t][kc];
                const vec8<T> b = oreg[t][kc];
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
                sc[kc] = acc;
            }
#pragma unroll
            for (int w = DV / 32; w >= 1; w /= 2) {
#pragma unroll
                for (int kc = 0; kc < w; ++kc) sc[kc] = sc[kc] + sc[kc + w];
            }
            nD[t] = -(sc[0] + xor_lane32(sc[0]));
            const float l = lraw[t];
            l2[t] = l > -INFINITY ? l * kLog2e : INFINITY;
            if (g == 0 && myq[t] < n_pad) {
                lse2[bh * (long)n_pad + myq[t]] = l2[t];
                Dw[bh * (long)n_pad + myq[t]] = nD[t];
            }
        }
    }
    // Q and dO rows are only MFMA inputs: keep them in AGPRs, leaving the
    // VGPRs to the S, dP and dS tiles of a 64-key step
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) asm volatile("" : "+a"(qreg[t][kc]));
#pragma unroll
        for (int kc = 0; kc < DV / 16; ++kc) asm volatile("" : "+a"(oreg[t][kc]));
    }

    TileOffsets<D> toK;
    toK.init(lane);
    TileOffsets<DV> toV;
    toV.init(lane);

    f32x16 acc[D / 32][2];
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
        acc[x][0] = zero16();
        acc[x][1] = zero16();
    }

    // One key tile (two 32-key halves kh) as a fixed sequence of operand
    // fragments, each read once from LDS and used by two MFMAs (query tiles
    // 0 and 1):
    //   f < FV:   K rows of half kh, d chunk r    -> S^T[kh][t]  += K Q_t^T
    //   f < FT:   V rows of half kh, dv chunk r   -> dP^T[kh][t] += V dO_t^T
    //   f < NF:   K^T, 16-key chunk c, d block x  -> dQ^T[x][t] += K^T dS^T
    // P = exp2(S * scale * log2e - LSE2) is formed during the dP products,
    // dS = P (dP - D) for chunk 0 right after them and for chunk c+1 during
    // the dQ products of chunk c.
    auto compute = [&](auto buf_, auto masked_, int k0) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_)::value;
        const T* Ks = Kbuf(buf_);
        const T* Vs = Vbuf(buf_);
        constexpr int KA = D / 16, KB = DV / 16, NX = D / 32;
        constexpr int NKH = BN / 32, NC = 2 * NKH;
        constexpr int FV = NKH * KA, FT = FV + NKH * KB, NF = FT + NC * NX;

        auto load_frag = [&](auto f_) __attribute__((always_inline)) -> vec8<T> {
            constexpr int f = decltype(f_)::value;
            if constexpr (f < FV) {
                return tile_read8_at<D>(Ks, toK, 32 * (f / KA), f % KA);
            } else if constexpr (f < FT) {
                return tile_read8_at<DV>(Vs, toV, 32 * ((f - FV) / KB), (f - FV) % KB);
            } else {
                constexpr int cx = f - FT, c = cx / NX, x = cx % NX;
                return tile_read_tr_at<D>(Ks, toK, 16 * c, x);
            }
        };

        f32x16 S[NKH][2], dP[NKH][2];
        vec8<T> dSb[NKH][2][2];

        int lim[2];
        if constexpr (MASKED) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                lim[t] = mb - 1 - k0 - 4 * g;
                if constexpr (CAUSAL) lim[t] = min(lim[t], myq[t] + off - k0 - 4 * g);
            }
        }
        // P for slot e of tile (kh, t), written over S; key k0 + 32kh + 4g +
        // 8(e>>2) + (e&3), visible when 32kh + 8(e>>2) + (e&3) <= lim[t].
        auto p_elem = [&](auto i_) __attribute__((always_inline)) {
            constexpr int i = decltype(i_)::value;
            constexpr int kh = i / 32, t = (i / 16) % 2, e = i % 16;
            float pv = fast_exp2(__builtin_fmaf(S[kh][t][e], c2, -l2[t]));
            if constexpr (MASKED) pv = (32 * kh + 8 * (e >> 2) + (e & 3) > lim[t]) ? 0.f : pv;
            S[kh][t][e] = pv;
        };
        // dS for 16-key chunk c of query tile t (row-of-C order operand).
        auto ds_chunk = [&](auto c_, auto t_) __attribute__((always_inline)) {
            constexpr int c = decltype(c_)::value, t = decltype(t_)::value;
            constexpr int kh = c / 2, h = c % 2;
            float d8[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                d8[s] = S[kh][t][8 * h + s] * dP[kh][t][8 * h + s];
            dSb[kh][t][h] = pack8<T>(d8[0], d8[1], d8[2], d8[3], d8[4], d8[5], d8[6], d8[7]);
        };

        vec8<T> fr[PD];
        static_for<PD>([&](auto f_) { fr[decltype(f_)::value] = load_frag(f_); });
        __builtin_amdgcn_sched_barrier(0);

        static_for<NF>([&](auto f_) {
            constexpr int f = decltype(f_)::value;
            const vec8<T> cur = fr[f % PD];
            if constexpr (f + PD < NF) fr[f % PD] = load_frag(std::integral_constant<int, f + PD>{});
            if constexpr (f < FV) {
                constexpr int kh = f / KA, r = f % KA;
                static_for<2>([&](auto t_) {
                    constexpr int t = decltype(t_)::value;
                    if constexpr (r == 0) S[kh][t] = zero16();
                    S[kh][t] = mfma32(cur, qreg[t][r], S[kh][t]);
                });
            } else if constexpr (f < FT) {
                constexpr int kh = (f - FV) / KB, r = (f - FV) % KB;
                static_for<2>([&](auto t_) {
                    constexpr int t = decltype(t_)::value;
                    // dP^T starts at -D: every slot of this lane is query myq[t]
                    if constexpr (r == 0) {
                        f32x16 start;
#pragma unroll
                        for (int e = 0; e < 16; ++e) start[e] = nD[t];
                        dP[kh][t] = mfma32(cur, oreg[t][0], start);
                    } else {
                        dP[kh][t] = mfma32(cur, oreg[t][r], dP[kh][t]);
                    }
                });
                // 32 NKH exponentials over the NKH KB dP slots
                static_for<32 * NKH>([&](auto i_) {
                    constexpr int i = decltype(i_)::value;
                    if constexpr ((i * KB) / 32 == f - FV) p_elem(i_);
                });
                if constexpr (f == FT - 1) {
                    ds_chunk(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
                    ds_chunk(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
                }
            } else {
                constexpr int cx = f - FT, c = cx / NX, x = cx % NX;
                static_for<2>([&](auto t_) {
                    constexpr int t = decltype(t_)::value;
                    mfma32_agpr<kOperandWait>(cur, dSb[c / 2][t][c % 2], acc[x][t]);
                });
                // dS of chunk c + 1 during the products of chunk c
                if constexpr (c + 1 < NC && x == 0)
                    ds_chunk(std::integral_constant<int, c + 1>{}, std::integral_constant<int, 0>{});
                if constexpr (c + 1 < NC && x == (NX > 1 ? 1 : 0))
                    ds_chunk(std::integral_constant<int, c + 1>{}, std::integral_constant<int, 1>{});
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    using MaskOn = std::integral_constant<bool, true>;
    using MaskOff = std::integral_constant<bool, false>;

    auto do_step = [&](auto buf_, auto masked_, int s) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_)::value;
        const int k0 = s * BN;
        if (s + 1 < nsteps) stage(std::integral_constant<int, buf ^ 1>{}, k0 + BN);
        compute(buf_, masked_, k0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Both loops start on buffer 0: an odd plain step joins the masked ones.
    const int n_plain2 = n_plain & ~1;
    int s = 0;
    for (; s < n_plain2; s += 2) {
        do_step(B0{}, MaskOff{}, s);
        do_step(B1{}, MaskOff{}, s + 1);
    }
    for (; s + 1 < nsteps; s += 2) {
        do_step(B0{}, MaskOn{}, s);
        do_step(B1{}, MaskOn{}, s + 1);
    }
    if (s < nsteps) do_step(B0{}, MaskOn{}, s);

    // wait states between the last MFMA writing an accumulator and the
    // reads below, and no read of an accumulator before them
    mfma_agpr_wait();
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
        mfma_agpr_fence(acc[x][0]);
        mfma_agpr_fence(acc[x][1]);
    }
    // Accumulator slot vv of tile (x, t) holds column d = 32x + 8(vv>>2) +
    // 4g + (vv&3) of query myq[t].  The tiles go out through this wave's
    // staging rows in LDS: written row-major (16-byte chunks XOR-swizzled by
    // row), read back as whole rows and stored 16 bytes per lane, eight
    // 128-byte row segments per instruction.
    if (dqacc != nullptr) {
        // float32 partial sums, 32 columns (128 bytes) per staged row; the
        // chunk swizzle by (row >> 1) & 7 keeps both the 16-byte writes (16
        // rows per lane group) and the row reads free of bank conflicts
        float* regf = reinterpret_cast<float*>(sE) + wave * 64 * 32;
        const __amdgpu_buffer_rsrc_t racc =
            make_rsrc(dqacc + bh * (long)n_pad * D, (uint32_t)(n_pad * D * 4));
#pragma unroll
        for (int x = 0; x < D / 32; ++x) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = 32 * t + li;
#pragma unroll
                for (int vq = 0; vq < 4; ++vq) {
                    const int chunk = 2 * vq + g;
                    *reinterpret_cast<f32x4*>(regf + row * 32 + 4 * (chunk ^ ((row >> 1) & 7))) =
                        f32x4{acc[x][t][4 * vq], acc[x][t][4 * vq + 1], acc[x][t][4 * vq + 2],
                              acc[x][t][4 * vq + 3]};
                }
            }
            f32x4 w4[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int lin = 64 * i + lane, row = lin >> 3, chunk = lin & 7;
                w4[i] = *reinterpret_cast<const f32x4*>(
                    regf + row * 32 + 4 * (chunk ^ ((row >> 1) & 7)));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int lin = 64 * i + lane, row = lin >> 3, chunk = lin & 7;
                const int query = i0 + (C::BM / 2) * (row / 32) + 32 * wave + row % 32;
                // rows at or past n_pad fall beyond the buffer and are dropped
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, w4[i]), racc,
                    (uint32_t)(((long)query * D + 32 * x + 4 * chunk) * 4), 0, 0);
            }
        }
        return;
    }
    T* reg = sE + wave * 64 * 64;
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc(dq + hq.base, (uint32_t)(n * hq.stride * 2));
#pragma unroll
    for (int sl = 0; sl < D / 64; ++sl) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = 32 * t + li;
#pragma unroll
            for (int xs = 0; xs < 2; ++xs) {
#pragma unroll
                for (int vq = 0; vq < 4; ++vq) {
                    vec4<T> w;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        w[r] = (T)(acc[2 * sl + xs][t][4 * vq + r] * scale);
                    const int chunk = 4 * xs + vq;
                    *reinterpret_cast<vec4<T>*>(reg + row * 64 + 8 * (chunk ^ (row & 7)) + 4 * g) = w;
                }
            }
        }
        vec8<T> w8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int lin = 64 * i + lane, row = lin / 8, chunk = lin % 8;
            w8[i] = *reinterpret_cast<const vec8<T>*>(reg + row * 64 + 8 * (chunk ^ (row & 7)));
        }
        // rows at or past n fall beyond the buffer, columns past dg get an
        // offset beyond it: the hardware drops both
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int lin = 64 * i + lane, row = lin / 8, chunk = lin % 8;
            const int query = i0 + (C::BM / 2) * (row / 32) + 32 * wave + row % 32;
            const int col = 64 * sl + 8 * chunk;
            const uint32_t byte_off =
                col < dg ? (uint32_t)(((long)query * hq.stride + col) * 2) : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w8[i]), rdq,
                                                   byte_off, 0, 0);
        }
    }
}

template <typename T, int D, int DV>
void launch_dq(const Problem& p, const void* q, const void* k, const void* v, const void* dout,
               const void* o, const float* lse, const Workspace& w, void* dq, float* dqacc,
               int key_limit, hipStream_t s) {
    using C = DqCfg<D, DV>;
    dim3 grid((unsigned)p.heads(), (unsigned)((p.n + C::BM - 1) / C::BM));
    const float c2 = p.scale * kLog2e;
    const SeqInfo si = seq_info(p);
    if (p.causal)
        bwd_dq_kernel<T, D, DV, true><<<grid, 64 * C::NW, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (const T*)dout, w.lse2, w.D, (const T*)o,
            lse, (T*)dq, dqacc, key_limit, p.n, p.m, p.d, p.dv, w.n_pad, p.scale, c2, si);
    else
        bwd_dq_kernel<T, D, DV, false><<<grid, 64 * C::NW, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (const T*)dout, w.lse2, w.D, (const T*)o,
            lse, (T*)dq, dqacc, key_limit, p.n, p.m, p.d, p.dv, w.n_pad, p.scale, c2, si);
}

// dQ = scale * dqacc in T, for the rows i < n of every head (the
// accumulator's padded rows and columns are not copied); one thread per
// eight columns.
template <typename T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ dqacc,
                                                         T* __restrict__ dq, int n, int n_pad,
                                                         int acc_w, int dg, float scale,
                                                         long total, SeqInfo si) {
    const long id = (long)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int cpr = dg / 8;
    const long rowid = id / cpr;
    const int c8 = (int)(id - rowid * cpr);
    const long bh = rowid / n;
    const int i = (int)(rowid - bh * n);
    const float* src = dqacc + (bh * (long)n_pad + i) * acc_w + 8 * c8;
    const f32x4 a = *reinterpret_cast<const f32x4*>(src);
    const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
    const HeadView hv = head_view(si, bh, n, dg);
    *reinterpret_cast<vec8<T>*>(dq + hv.base + (long)i * hv.stride + 8 * c8) =
        pack8<T>(a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale, b[0] * scale,
                 b[1] * scale, b[2] * scale, b[3] * scale);
}

}  // namespace

template <typename T>
bool launch_bwd_dq_mfma(const Problem& p, const void* q, const void* k, const void* v,
                        const void* dout, const void* o, const float* lse, const Workspace& w,
                        void* dq, float* dqacc, int key_limit, hipStream_t s) {
    switch (mfma_widths(p)) {
    case 0x4040: launch_dq<T, 64, 64>(p, q, k, v, dout, o, lse, w, dq, dqacc, key_limit, s); break;
    case 0x4080: launch_dq<T, 64, 128>(p, q, k, v, dout, o, lse, w, dq, dqacc, key_limit, s); break;
    case 0x8040: launch_dq<T, 128, 64>(p, q, k, v, dout, o, lse, w, dq, dqacc, key_limit, s); break;
    case 0x8080: launch_dq<T, 128, 128>(p, q, k, v, dout, o, lse, w, dq, dqacc, key_limit, s); break;
    default: return false;
    }
    return true;
}

template <typename T>
void launch_dq_convert(const Problem& p, const Workspace& w, void* dq, hipStream_t s) {
    const long total = p.heads() * (long)p.n * (p.d / 8);
    if (total == 0) return;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    dq_convert_kernel<T><<<blocks, 256, 0, s>>>(w.dqacc, (T*)dq, p.n, w.n_pad, w.acc_w, p.d,
                                                p.scale, total, seq_info(p));
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template bool launch_bwd_dq_mfma<ATTN_ELEM>(const Problem&, const void*, const void*,
                                           const void*, const void*, const void*, const float*,
                                           const Workspace&, void*, float*, int, hipStream_t);
template void launch_dq_convert<ATTN_ELEM>(const Problem&, const Workspace&, void*, hipStream_t);

}  // namespace attn

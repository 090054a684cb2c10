// Forward attention on 16-bit MFMA (bf16 or f16 inputs, float32
// accumulation and softmax statistics); emits O
// and the per-row log-sum-exp that the backward uses to recompute P
// (mlgrind "Forward"; "Attention Backpropagation: Step by step
// derivation", section Forward Pass).
//
// Layout: one workgroup per 256 queries of a head, four waves, each wave
// owning two 32-query MFMA tiles.  The lane owns a query column of the
// transposed products
//     S^T = K Q^T,   O^T += V^T P^T,
// so this lane's row of Q is a register-resident B operand, the online
// row max and row sum are per-lane values (plus one exchange with the
// lane 32 away, which holds the other half of the keys), and P^T in
// accumulator layout is the B operand of the O product in row-of-C order
// (see attn_device.h).  Every 64-key tile of K and V is staged once in LDS
// and each fragment read from it feeds two MFMAs, one per query tile.
//
// The running max is raised lazily: the accumulators and the row sum are
// rescaled only when some row's max grows by more than 2^8 (in the base-2
// domain), so P = exp2(S * scale * log2e - m) stays below 2^8 and the
// rescale, which touches every accumulator, is rare; so is the exchange of
// the two lanes' maxima that a rescale needs.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D, int DV>
struct FwdCfg {
    static constexpr int NW = 4;              // waves per workgroup
    static constexpr int BM = 2 * 32 * NW;    // queries per workgroup
    static constexpr int BN = 64;             // keys per step
    static constexpr int PD = 4;              // operand reads issued ahead
};

constexpr float kRescaleThreshold = 8.f;     // log2 of the largest P allowed

template <typename T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ o, float* __restrict__ lse, int n, int m, int dg, int dvg, float c2,
    SeqInfo si) {
    using C = FwdCfg<D, DV>;
    constexpr int BN = C::BN, PD = C::PD, NW = C::NW;
    constexpr int KA = D / 16, NXV = DV / 32;
    // One LDS variable per buffer: reads of one buffer are then known not
    // to alias the asynchronous fills of the other.
    __shared__ __align__(1024) T sK0[BN * D];
    __shared__ __align__(1024) T sK1[BN * D];
    __shared__ __align__(1024) T sV0[BN * DV];
    __shared__ __align__(1024) T sV1[BN * DV];
    // the epilogue's staging rows: 64 rows x 64 columns per wave
    __shared__ __align__(1024) T sE[NW * 64 * 64];
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
    const int qb = CAUSAL ? (int)gridDim.y - 1 - to.rank : to.rank;
    const int i0 = qb * C::BM;
    // This head's query and key lengths and causal offset: rows i < nb take
    // part, keys j < mb, and key j is visible from row i when j <= i + off.
    const SeqLens len = seq_lens(si, bh, n, m);
    const int nb = len.n, mb = len.m, off = len.off;

    // Rows of Q and K hold dg <= D elements, rows of V and O dvg <= DV (each
    // a multiple of 8); the columns past them are zeros in registers and
    // LDS, so they add nothing to any product.
    const HeadView hq = head_view(si, bh, n, dg), hk = head_view(si, bh, m, dg);
    const HeadView hv = head_view(si, bh, m, dvg), ho = head_view(si, bh, n, dvg);
    const T* qh = q + hq.base;
    const T* kh = k + hk.base;
    const T* vh = v + hv.base;

    // A negative scale is handled by negating Q, so that the row max of
    // S * c2 is c2 times the row max of the computed S.  A zero scale is
    // raised to 1e-30, so that masked logits (-inf) stay -inf after the
    // multiplication (-inf * 0 would be NaN); 1e-30 times a finite logit is
    // far below float32 resolution at 1, so every visible weight is exactly
    // 1, as with a zero scale.
    const bool neg = c2 < 0.f;
    const float cs = fmaxf(neg ? -c2 : c2, 1e-30f);

    // Query tile t of this wave: rows i0 + (BM/2) t + 32 wave + (0..31), one
    // tile from each half of the workgroup's rows (even causal work).
    int myq[2];
    vec8<T> qreg[2][KA];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        myq[t] = i0 + (C::BM / 2) * t + 32 * wave + li;
        const bool ok = myq[t] < nb;
#pragma unroll
        for (int kc = 0; kc < KA; ++kc) {
            const bool in = ok && 16 * kc + 8 * g < dg;
            vec8<T> x = in ? gload8(qh + (long)myq[t] * hq.stride + 16 * kc + 8 * g) : vec8<T>{};
            if (neg) x = __builtin_bit_cast(vec8<T>, __builtin_bit_cast(u32x4, x) ^ 0x80008000u);
            qreg[t][kc] = x;
            // keep the Q operands in AGPRs (MFMAs read them from there), so
            // that the VGPRs hold the four S tiles of a step
            asm volatile("" : "+a"(qreg[t][kc]));
        }
    }

    TileOffsets<D> toK;
    toK.init(lane);
    TileOffsets<DV> toV;
    toV.init(lane);

    // Keys below k_end reach some row of the workgroup; the first n_plain
    // steps are visible from all of its rows and need no mask.
    int k_end = CAUSAL ? min(mb, i0 + C::BM + off) : mb;
    if (i0 >= nb) k_end = 0;
    const int nsteps = (max(k_end, 0) + BN - 1) / BN;
    int n_plain = min(nsteps, mb / BN);
    if (CAUSAL) n_plain = min(n_plain, max(i0 + off + 1, 0) / BN);

    // Key tiles go to LDS buffer s & 1 for step s, fetched one step ahead;
    // rows past mb come back as zeros and are masked.
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(kh, (uint32_t)mb * hk.stride * 2);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(vh, (uint32_t)mb * hv.stride * 2);
    TileLoader<D, BN, NW> ldK;
    ldK.init(wave, lane, dg, hk.stride);
    TileLoader<DV, BN, NW> ldV;
    ldV.init(wave, lane, dvg, hv.stride);
    auto stage = [&](auto buf_, int k0) __attribute__((always_inline)) {
        tile_fill<D, BN, NW>(ldK, pick(buf_, sK0, sK1), rK, k0, wave);
        tile_fill<DV, BN, NW>(ldV, pick(buf_, sV0, sV1), rV, k0, wave);
    };

    // O^T accumulators, running max (base 2) and this lane's part of the
    // running sum, per query tile.  The accumulators stay in VGPRs: the
    // rare rescale multiplies them in place, where AGPR accumulators made
    // the compiler copy all 128 of them to VGPRs at the top of every step
    // (about 7% of the kernel's time at 4k context).
    f32x16 acc[NXV][2];
#pragma unroll
    for (int x = 0; x < NXV; ++x) {
        acc[x][0] = zero16();
        acc[x][1] = zero16();
    }
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    // One key tile: fragments f < NKH KA are K rows of 32-key half kh
    // (S^T[kh][t] += K Q_t^T, two MFMAs each); then the softmax; then
    // fragments (c, x) of V^T for O^T[x][t] += V^T P^T[t] over 16-key chunk
    // c, two MFMAs each.  The exponentials of chunk c+1 run during the
    // products of chunk c.
    auto compute = [&](auto buf_, auto masked_, int k0) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_)::value;
        constexpr int NKH = BN / 32;                    // 32-key halves per step
        constexpr int NC = 2 * NKH;                     // 16-key chunks per step
        const T* Ks = pick(buf_, sK0, sK1);
        const T* Vs = pick(buf_, sV0, sV1);
        constexpr int NF = NKH * KA + NC * NXV;

        auto load_frag = [&](auto f_) __attribute__((always_inline)) -> vec8<T> {
            constexpr int f = decltype(f_)::value;
            if constexpr (f < NKH * KA) {
                return tile_read8_at<D>(Ks, toK, 32 * (f / KA), f % KA);
            } else {
                constexpr int cx = f - NKH * KA, c = cx / NXV, x = cx % NXV;
                return tile_read_tr_at<DV>(Vs, toV, 16 * c, x);
            }
        };

        f32x16 S[NKH][2];
        vec8<T> Pb[NC][2];
        float mbase[2];   // running max used as the exponent base
        int lim[2];
        if constexpr (MASKED) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                lim[t] = mb - 1 - k0 - 4 * g;
                if constexpr (CAUSAL) lim[t] = min(lim[t], myq[t] + off - k0 - 4 * g);
            }
        }
        // Masked steps set the invisible logits to -inf once, before the
        // row max; exp2 then gives their P = 0 with no second test (one
        // compare per element, consumed at once, instead of 64 lane masks
        // kept for the P pass, which spilled scalar registers).
        auto visible = [&](int kh, int e, int t) __attribute__((always_inline)) {
            return 32 * kh + 8 * (e >> 2) + (e & 3) <= lim[t];
        };
        // The row max is only needed when it grows past the threshold, and
        // it grows past it exactly when this lane's half of the keys or the
        // other lane's half does: each lane tests its own half, and only
        // when some lane of the wave sees growth are the halves exchanged
        // (a round trip through LDS) and the running max raised.
        auto softmax_head = [&]() __attribute__((always_inline)) {
            float mx[2];
            bool grow = false;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                mx[t] = -INFINITY;
#pragma unroll
                for (int kh = 0; kh < NKH; ++kh) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        if constexpr (MASKED)
                            S[kh][t][e] = visible(kh, e, t) ? S[kh][t][e] : -INFINITY;
                        mx[t] = fmaxf(mx[t], S[kh][t][e]);
                    }
                }
                grow |= mx[t] != -INFINITY && mx[t] * cs > m_run[t] + kRescaleThreshold;
            }
            if (__any(grow)) {
                float m_new[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const float m2 = fmaxf(mx[t], xor_lane32(mx[t]));
                    m_new[t] = m2 == -INFINITY ? m_run[t] : fmaxf(m_run[t], m2 * cs);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const float alpha = m_new[t] == m_run[t] ? 1.f : fast_exp2(m_run[t] - m_new[t]);
                    l_run[t] *= alpha;
#pragma unroll
                    for (int x = 0; x < NXV; ++x) acc[x][t] *= alpha;
                    m_run[t] = m_new[t];
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) mbase[t] = m_run[t] == -INFINITY ? 0.f : m_run[t];
        };
        auto p_chunk = [&](auto c_, auto t_) __attribute__((always_inline)) {
            constexpr int c = decltype(c_)::value, t = decltype(t_)::value;
            constexpr int kh = c / 2, e0 = 8 * (c % 2);
            float p8[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                float pv = fast_exp2(__builtin_fmaf(S[kh][t][e0 + s], cs, -mbase[t]));
                p8[s] = pv;
                l_run[t] += pv;
            }
            Pb[c][t] = pack8<T>(p8[0], p8[1], p8[2], p8[3], p8[4], p8[5], p8[6], p8[7]);
        };

        vec8<T> fr[PD];
        static_for<PD>([&](auto f_) { fr[decltype(f_)::value] = load_frag(f_); });
        __builtin_amdgcn_sched_barrier(0);

        static_for<NF>([&](auto f_) {
            constexpr int f = decltype(f_)::value;
            const vec8<T> cur = fr[f % PD];
            if constexpr (f + PD < NF) fr[f % PD] = load_frag(std::integral_constant<int, f + PD>{});
            if constexpr (f < NKH * KA) {
                constexpr int kh = f / KA, r = f % KA;
                static_for<2>([&](auto t_) {
                    constexpr int t = decltype(t_)::value;
                    if constexpr (r == 0) S[kh][t] = zero16();
                    S[kh][t] = mfma32(cur, qreg[t][r], S[kh][t]);
                });
                if constexpr (f == NKH * KA - 1) {
                    softmax_head();
                    p_chunk(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
                    p_chunk(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
                }
            } else {
                constexpr int cx = f - NKH * KA, c = cx / NXV, x = cx % NXV;
                static_for<2>([&](auto t_) {
                    constexpr int t = decltype(t_)::value;
                    acc[x][t] = mfma32(cur, Pb[c][t], acc[x][t]);
                });
                // chunk c + 1 while the products of chunk c run
                if constexpr (c + 1 < NC && x == 0)
                    p_chunk(std::integral_constant<int, c + 1>{}, std::integral_constant<int, 0>{});
                if constexpr (c + 1 < NC && x == (NXV > 1 ? 1 : 0))
                    p_chunk(std::integral_constant<int, c + 1>{}, std::integral_constant<int, 1>{});
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
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

    if (nsteps > 0) stage(B0{}, 0);
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

    // Accumulator slot vv of tile (x, t) holds column 32x + 8(vv>>2) + 4g +
    // (vv&3) of query myq[t]; the row sum is split over this lane and the
    // lane 32 away.  Rows past nb, and rows that see no key (row sum 0),
    // are written as O = 0, LSE = -inf.  The O tiles go out through this
    // wave's staging rows in LDS, 64 columns at a time: written row-major
    // (16-byte chunks XOR-swizzled by row), read back as whole rows and
    // stored 16 bytes per lane, eight 128-byte row segments per instruction.
    float inv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float l_tot = l_run[t] + xor_lane32(l_run[t]);
        const bool seen = myq[t] < nb && l_tot > 0.f;
        inv[t] = seen ? 1.f / l_tot : 0.f;
        if (myq[t] < n && g == 0)
            lse[bh * (long)n + myq[t]] = seen ? (m_run[t] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
    T* reg = sE + wave * 64 * 64;
#pragma unroll
    for (int sl = 0; sl < DV / 64; ++sl) {
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
                        w[r] = (T)(acc[2 * sl + xs][t][4 * vq + r] * inv[t]);
                    const int chunk = 4 * xs + vq;
                    *reinterpret_cast<vec4<T>*>(reg + row * 64 + 8 * (chunk ^ (row & 7)) + 4 * g) = w;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int lin = 64 * i + lane, row = lin / 8, chunk = lin % 8;
            const vec8<T> w8 =
                *reinterpret_cast<const vec8<T>*>(reg + row * 64 + 8 * (chunk ^ (row & 7)));
            const int query = i0 + (C::BM / 2) * (row / 32) + 32 * wave + row % 32;
            const int col = 64 * sl + 8 * chunk;
            if (query < n && col < dvg)
                *reinterpret_cast<vec8<T>*>(o + ho.base + (long)query * ho.stride + col) = w8;
        }
    }
}

template <typename T, int D, int DV>
void launch(const Problem& p, const void* q, const void* k, const void* v, void* o,
            float* lse, hipStream_t s) {
    using C = FwdCfg<D, DV>;
    dim3 grid((unsigned)p.heads(), (unsigned)((p.n + C::BM - 1) / C::BM));
    const float c2 = p.scale * kLog2e;
    const SeqInfo si = seq_info(p);
    if (p.causal)
        fwd_kernel<T, D, DV, true><<<grid, 64 * C::NW, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, p.n, p.m, p.d, p.dv, c2, si);
    else
        fwd_kernel<T, D, DV, false><<<grid, 64 * C::NW, 0, s>>>(
            (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, p.n, p.m, p.d, p.dv, c2, si);
}

}  // namespace

template <typename T>
bool launch_fwd_mfma(const Problem& p, const void* q, const void* k, const void* v, void* o,
                     float* lse, hipStream_t s) {
    switch (mfma_widths(p)) {
    case 0x4040: launch<T, 64, 64>(p, q, k, v, o, lse, s); break;
    case 0x4080: launch<T, 64, 128>(p, q, k, v, o, lse, s); break;
    case 0x8040: launch<T, 128, 64>(p, q, k, v, o, lse, s); break;
    case 0x8080: launch<T, 128, 128>(p, q, k, v, o, lse, s); break;
    default: return false;
    }
    return true;
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template bool launch_fwd_mfma<ATTN_ELEM>(const Problem&, const void*, const void*, const void*,
                                        void*, float*, hipStream_t);

}  // namespace attn

// Forward attention on bf16 MFMA with float32 softmax statistics; emits O
// and the per-row log-sum-exp that the backward uses to recompute P.
//
// Per workgroup: 128 query rows of one (batch, head), 32 per wave.  Each
// step stages 64 keys: K row-major and V transposed in LDS (double
// buffered, next tile prefetched into registers during the current one).
// The wave computes S^T = K Q^T so that a lane owns one query: the online
// row max and row sum are per-lane values (plus one exchange with the lane
// 32 away), and P^T in accumulator layout feeds O^T += V^T P^T directly as
// the B operand (row-of-C order), with no trip through LDS.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

template <int D, int DV>
struct FwdCfg {
    static constexpr int BM = 128;          // queries per workgroup
    static constexpr int BN = 64;           // keys per step
    static constexpr int LDK = D + 8;       // row stride of K in LDS (elements)
    static constexpr int LDT = BN + 4;      // row stride of V^T in LDS
    static constexpr int K_ITEMS = BN * D / 8;            // 16-byte chunks of K
    static constexpr int VT_ITEMS = (BN / 4) * (DV / 8);  // 4x8 blocks of V
    static constexpr int K_PER_T = (K_ITEMS + 255) / 256;
    static constexpr int VT_PER_T = (VT_ITEMS + 255) / 256;
};

template <int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse, int n, int m, float c2) {
    using C = FwdCfg<D, DV>;
    __shared__ __align__(16) bf16 sK[2][C::BN * C::LDK];
    __shared__ __align__(16) bf16 sVT[2][DV * C::LDT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, li = lane & 31;
    const long bh = blockIdx.x;
    const int qb = CAUSAL ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
    const int i0 = qb * C::BM;
    const int myq = i0 + wave * 32 + li;

    const bf16* qh = q + bh * (long)n * D;
    const bf16* kh = k + bh * (long)m * D;
    const bf16* vh = v + bh * (long)m * DV;

    // This lane's query row as the B operand of S^T = K Q^T (natural k order).
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        if (myq < n) qreg[kc] = gload_bf16x8(qh + (long)myq * D + 16 * kc + 8 * g);
        else qreg[kc] = bf16x8{};
    }

    const int k_end = CAUSAL ? min(m, i0 + C::BM) : m;
    const int nsteps = (k_end + C::BN - 1) / C::BN;

    u32x4 kst[C::K_PER_T];
    u32x4 vst[C::VT_PER_T][4];

    auto fetch = [&](int k0) {
#pragma unroll
        for (int it = 0; it < C::K_PER_T; ++it) {
            const int e = tid + it * 256;
            if (e < C::K_ITEMS) {
                const int r = e / (D / 8), cg = e % (D / 8);
                const int key = k0 + r;
                kst[it] = key < m ? gload16(kh + (long)key * D + 8 * cg) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int it = 0; it < C::VT_PER_T; ++it) {
            const int e = tid + it * 256;
            if (e < C::VT_ITEMS) {
                const int rg = e / (DV / 8), cg = e % (DV / 8);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int key = k0 + 4 * rg + x;
                    vst[it][x] = key < m ? gload16(vh + (long)key * DV + 8 * cg)
                                         : u32x4{0, 0, 0, 0};
                }
            }
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int it = 0; it < C::K_PER_T; ++it) {
            const int e = tid + it * 256;
            if (e < C::K_ITEMS) {
                const int r = e / (D / 8), cg = e % (D / 8);
                lds_write16(&sK[buf][r * C::LDK + 8 * cg], kst[it]);
            }
        }
#pragma unroll
        for (int it = 0; it < C::VT_PER_T; ++it) {
            const int e = tid + it * 256;
            if (e < C::VT_ITEMS) {
                const int rg = e / (DV / 8), cg = e % (DV / 8);
#pragma unroll
                for (int y = 0; y < 8; ++y)
                    lds_write8(&sVT[buf][(8 * cg + y) * C::LDT + 4 * rg], column4(vst[it], y));
            }
        }
    };

    f32x16 acc[DV / 32];
#pragma unroll
    for (int mt = 0; mt < DV / 32; ++mt) acc[mt] = zero16();
    float m_run = -INFINITY, l_run = 0.f;

    if (nsteps > 0) {
        fetch(0);
        commit(0);
    }
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        const int k0 = step * C::BN;
        const bool has_next = step + 1 < nsteps;
        if (has_next) fetch(k0 + C::BN);

        const bf16* Ks = sK[buf];
        const bf16* VTs = sVT[buf];
        f32x16 S[2];
        S[0] = zero16();
        S[1] = zero16();
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 a = lds_read8(Ks + (32 * t + li) * C::LDK + 16 * kc + 8 * g);
                S[t] = mfma32(a, qreg[kc], S[t]);
            }
        }

        const bool need_mask = (CAUSAL && k0 + C::BN - 1 > i0) || (k0 + C::BN > m);
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                float sv = S[t][vv] * c2;
                if (need_mask) {
                    const int key = k0 + 32 * t + 8 * (vv >> 2) + 4 * g + (vv & 3);
                    if (key >= m || (CAUSAL && key > myq)) sv = -INFINITY;
                }
                S[t][vv] = sv;
                mx = fmaxf(mx, sv);
            }
        }
        mx = fmaxf(mx, xor_lane32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float base = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - base);
        float psum = 0.f;
        bf16x8 Pb[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float p[16];
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                p[vv] = fast_exp2(S[t][vv] - base);
                psum += p[vv];
            }
            Pb[t][0] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
            Pb[t][1] = pack8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int mt = 0; mt < DV / 32; ++mt) {
            acc[mt] = acc[mt] * alpha;
            const bf16* row = VTs + (32 * mt + li) * C::LDT;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    bf16x8 a = read_rowc_pair(row, 32 * t + 16 * c, g);
                    acc[mt] = mfma32(a, Pb[t][c], acc[mt]);
                }
            }
        }

        if (has_next) commit(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + xor_lane32(l_run);
    const float inv = 1.f / l_tot;
    if (myq < n) {
        bf16* orow = o + (bh * (long)n + myq) * DV;
#pragma unroll
        for (int mt = 0; mt < DV / 32; ++mt) {
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(acc[mt][4 * vq + r] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * mt + 8 * vq + 4 * g) = w;
            }
        }
        if (g == 0) lse[bh * (long)n + myq] = (m_run + log2f(l_tot)) * kLn2;
    }
}

template <int D, int DV>
void launch(const Problem& p, const void* q, const void* k, const void* v, void* o,
            float* lse, hipStream_t s) {
    using C = FwdCfg<D, DV>;
    dim3 grid((unsigned)p.heads(), (unsigned)((p.n + C::BM - 1) / C::BM));
    const float c2 = p.scale * kLog2e;
    if (p.causal)
        fwd_bf16_kernel<D, DV, true><<<grid, 256, 0, s>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, p.n, p.m, c2);
    else
        fwd_bf16_kernel<D, DV, false><<<grid, 256, 0, s>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, p.n, p.m, c2);
}

}  // namespace

bool launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o,
                     float* lse, hipStream_t s) {
    if (p.d == 64 && p.dv == 64) launch<64, 64>(p, q, k, v, o, lse, s);
    else if (p.d == 128 && p.dv == 128) launch<128, 128>(p, q, k, v, o, lse, s);
    else if (p.d == 128 && p.dv == 64) launch<128, 64>(p, q, k, v, o, lse, s);
    else return false;
    return true;
}

}  // namespace attn

// Dense products of the layer around attention: the projection gradients
// of a multi-head self-attention layer (eulerpad "Attention backward"
// Problems 7 and 10; datatweets "Step 4: Back to the Parameters and
// Input").  With tokens as rows (batch and sequence flattened; the
// [B, seq, H, dim] attention layout is exactly this [T, H dim] matrix):
//
//   out projection  Y = O_cat W_O:   dW_O = O_cat^T G      (TN)
//                                    dO_cat = G W_O^T      (NT)
//   in projections  Q = X W_Q, ...:  dW_P = X^T dP_cat     (TN, P = Q, K, V)
//                                    dX = sum_P dP_cat W_P^T   (NT, three products)
//
// Two kernels, both 16-bit inputs with float32 accumulation:
//   NT: C[M, N] = sum_p A_p[M, K_p] B_p[N, K_p]^T   (rows of A and B run along k)
//   TN: C[M, N] = A[K, M]^T B[K, N]                 (rows of A and B run along m, n)
//
// Layout: a 256 x 256 tile of C per workgroup, four waves as 2 x 2, each
// wave 128 x 128 = 4 x 4 MFMA tiles of 32 x 32 whose accumulators (256
// registers) live in AGPRs.  k advances 64 at a time; both operand tiles of
// the next step are fetched by buffer loads straight into the other LDS
// buffer while the current step's 64 MFMAs per wave run.  Every operand
// fragment read from LDS feeds four MFMAs.  NT tiles are stored as read
// (256 rows of 64 k) and read in natural k order; TN tiles (64 rows of k,
// 128 columns per half) are read with the transposing LDS read, which
// gives both operands the same row-of-C k order.  Out-of-range rows and
// columns load as zeros (buffer bounds, or chunk offsets past the end) and
// are not stored.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int GBM = 256, GBN = 256, GBK = 64, GNW = 4;

// Fill a tile through a loader whose offsets are relative to element
// `base` of the buffer behind rsrc.
template <int C, int ROWS, int NW, typename T>
__device__ __forceinline__ void tile_fill_at(const TileLoader<C, ROWS, NW>& L, T* lds_tile,
                                             __amdgpu_buffer_rsrc_t rsrc, long base, int w) {
#pragma unroll
    for (int jj = 0; jj < TileLoader<C, ROWS, NW>::N; ++jj)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(lds_tile + (w + NW * jj) * 512),
                                                 16, (unsigned)(2 * L.off[jj]),
                                                 (unsigned)(2 * base), 0, 0);
}

// Which C tile this workgroup computes.  Workgroups are dealt to the eight
// XCDs in turn, so consecutive tile numbers are given to one XCD; tiles are
// numbered in groups of 8 row tiles, column-major inside a group, so that
// the workgroups sharing an XCD's L2 share A and B panels.
__device__ __forceinline__ bool pick_tile(int tm, int tn, int& mt, int& nt) {
    const int tiles = tm * tn, per = (tiles + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= tiles) return false;
    const int group = t / (8 * tn), first = 8 * group;
    const int gm = min(tm - first, 8), r = t - group * 8 * tn;
    mt = first + r % gm;
    nt = r / gm;
    return true;
}

// Store a wave's 128 x 128 block: accumulator (i, j) slot v holds row
// 32i + 8(v>>2) + 4g + (v&3), column 32j + li of the block.
template <typename OutT>
__device__ __forceinline__ void store_block(OutT* c, long ldc, int M, int N, int row0, int col0,
                                            f32x16 (&acc)[4][4], int g, int li) {
    // (no per-accumulator fence here: it made the register allocator copy
    // accumulators at the loop exit, before the wait; the build's hazard
    // check confirms that every accumulator read follows the wait)
    mfma_agpr_wait();
    OutT* base = c + (long)(row0 + 4 * g) * ldc + col0 + li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = 32 * i + 8 * (v >> 2) + (v & 3);   // row - row0 - 4g
            if (row0 + 4 * g + r >= M) continue;
            OutT* rowp = base + (long)r * ldc;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (col0 + 32 * j + li < N) rowp[32 * j] = (OutT)acc[i][j][v];
        }
    }
}

// ------------------------------------------------------------------- NT

struct NTArgs {
    const void* a[3];   // A_p [M, K_p], rows lda_p apart
    const void* b[3];   // B_p [N, K_p], rows ldb_p apart
    int k[3], lda[3], ldb[3];
    int count;          // number of products (1..3)
};

template <typename T, typename OutT>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_nt_kernel(
    NTArgs args, OutT* __restrict__ c, long ldc, int M, int N, int tm, int tn) {
    __shared__ __align__(1024) T sA0[GBM * GBK];
    __shared__ __align__(1024) T sA1[GBM * GBK];
    __shared__ __align__(1024) T sB0[GBN * GBK];
    __shared__ __align__(1024) T sB1[GBN * GBK];
    auto pick = [](auto b_, auto* x0, auto* x1) __attribute__((always_inline)) {
        if constexpr (decltype(b_)::value == 0) return x0;
        else return x1;
    };
    int mt, nt;
    if (!pick_tile(tm, tn, mt, nt)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: a scalar register
    const int g = lane >> 5, li = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = mt * GBM, n0 = nt * GBN;

    TileOffsets<GBK> to;
    to.init(lane);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero16();

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    for (int p = 0; p < args.count; ++p) {
        const T* A = (const T*)args.a[p];
        const T* Bm = (const T*)args.b[p];
        const int K = args.k[p], lda = args.lda[p], ldb = args.ldb[p];
        const int nsteps = (K + GBK - 1) / GBK;
        // rows past M (N) lie past the buffer's end and load as zeros
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + (long)m0 * lda, (uint32_t)(max(M - m0, 0)) * lda * 2);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bm + (long)n0 * ldb, (uint32_t)(max(N - n0, 0)) * ldb * 2);
        TileLoader<GBK, GBM, GNW> ldA, ldB;
        ldA.init(wave, lane, GBK, lda);
        ldB.init(wave, lane, GBK, ldb);
        // the last step may hold fewer than 64 k: chunks past K load zeros
        auto stage = [&](auto buf_, int s) __attribute__((always_inline)) {
            const int k0 = s * GBK;
            if (k0 + GBK > K) {
                ldA.init(wave, lane, K - k0, lda);
                ldB.init(wave, lane, K - k0, ldb);
            }
            tile_fill_at(ldA, pick(buf_, sA0, sA1), rA, k0, wave);
            tile_fill_at(ldB, pick(buf_, sB0, sB1), rB, k0, wave);
        };
        auto compute = [&](auto buf_) __attribute__((always_inline)) {
            const T* As = pick(buf_, sA0, sA1) + (wm * 128) * GBK;
            const T* Bs = pick(buf_, sB0, sB1) + (wn * 128) * GBK;
            vec8<T> fa[2][4], fb[2][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[0][i] = tile_read8_at<GBK>(As, to, 32 * i, 0);
                fb[0][i] = tile_read8_at<GBK>(Bs, to, 32 * i, 0);
            }
            static_for<GBK / 16>([&](auto kc_) {
                constexpr int kc = decltype(kc_)::value, cur = kc & 1;
                if constexpr (kc + 1 < GBK / 16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        fa[cur ^ 1][i] = tile_read8_at<GBK>(As, to, 32 * i, kc + 1);
                        fb[cur ^ 1][i] = tile_read8_at<GBK>(Bs, to, 32 * i, kc + 1);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mfma32_agpr(fa[cur][i], fb[cur][j], acc[i][j]);
            });
        };
        auto do_step = [&](auto buf_, int s) __attribute__((always_inline)) {
            constexpr int buf = decltype(buf_)::value;
            if (s + 1 < nsteps) stage(std::integral_constant<int, buf ^ 1>{}, s + 1);
            compute(buf_);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        if (nsteps > 0) stage(B0{}, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            do_step(B0{}, s);
            do_step(B1{}, s + 1);
        }
        if (s < nsteps) do_step(B0{}, s);
    }
    store_block(c, ldc, M, N, m0 + wm * 128, n0 + wn * 128, acc, g, li);
}

// ------------------------------------------------------------------- TN

template <typename T, typename OutT>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_tn_kernel(
    const T* __restrict__ A, int lda, const T* __restrict__ Bm, int ldb, OutT* __restrict__ c,
    long ldc, int M, int N, int K, int tm, int tn) {
    // [k][128] halves: sA*[h] holds columns m0 + 128h .. m0 + 128h + 127
    __shared__ __align__(1024) T sA0[2 * GBK * 128];
    __shared__ __align__(1024) T sA1[2 * GBK * 128];
    __shared__ __align__(1024) T sB0[2 * GBK * 128];
    __shared__ __align__(1024) T sB1[2 * GBK * 128];
    auto pick = [](auto b_, auto* x0, auto* x1) __attribute__((always_inline)) {
        if constexpr (decltype(b_)::value == 0) return x0;
        else return x1;
    };
    int mt, nt;
    if (!pick_tile(tm, tn, mt, nt)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: a scalar register
    const int g = lane >> 5, li = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = mt * GBM, n0 = nt * GBN;

    // rows past K lie past the buffer's end; columns past M (N) are masked
    // chunk by chunk
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(A, (uint32_t)K * lda * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bm, (uint32_t)K * ldb * 2);
    TileLoader<128, GBK, GNW> ldA[2], ldB[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ldA[h].init(wave, lane, min(max(M - m0 - 128 * h, 0), 128), lda);
        ldB[h].init(wave, lane, min(max(N - n0 - 128 * h, 0), 128), ldb);
    }
    TileOffsets<128> to;
    to.init(lane);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero16();

    const int nsteps = (K + GBK - 1) / GBK;
    auto stage = [&](auto buf_, int s) __attribute__((always_inline)) {
        const long k0 = (long)s * GBK;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            tile_fill_at(ldA[h], pick(buf_, sA0, sA1) + h * GBK * 128, rA,
                         k0 * lda + m0 + 128 * h, wave);
            tile_fill_at(ldB[h], pick(buf_, sB0, sB1) + h * GBK * 128, rB,
                         k0 * ldb + n0 + 128 * h, wave);
        }
    };
    auto compute = [&](auto buf_) __attribute__((always_inline)) {
        const T* As = pick(buf_, sA0, sA1) + wm * GBK * 128;
        const T* Bs = pick(buf_, sB0, sB1) + wn * GBK * 128;
        vec8<T> fa[2][4], fb[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[0][i] = tile_read_tr_at<128>(As, to, 0, i);
            fb[0][i] = tile_read_tr_at<128>(Bs, to, 0, i);
        }
        static_for<GBK / 16>([&](auto kc_) {
            constexpr int kc = decltype(kc_)::value, cur = kc & 1;
            if constexpr (kc + 1 < GBK / 16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fa[cur ^ 1][i] = tile_read_tr_at<128>(As, to, 16 * (kc + 1), i);
                    fb[cur ^ 1][i] = tile_read_tr_at<128>(Bs, to, 16 * (kc + 1), i);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mfma32_agpr(fa[cur][i], fb[cur][j], acc[i][j]);
        });
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto do_step = [&](auto buf_, int s) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_)::value;
        if (s + 1 < nsteps) stage(std::integral_constant<int, buf ^ 1>{}, s + 1);
        compute(buf_);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    if (nsteps > 0) stage(B0{}, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        do_step(B0{}, s);
        do_step(B1{}, s + 1);
    }
    if (s < nsteps) do_step(B0{}, s);
    store_block(c, ldc, M, N, m0 + wm * 128, n0 + wn * 128, acc, g, li);
}

template <typename T, typename OutT>
void launch_nt(const NTArgs& args, void* c, long ldc, int M, int N, hipStream_t s) {
    const int tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
    if (tm * tn == 0) return;   // no rows (T = 0): nothing to write
    const unsigned grid = 8u * (unsigned)((tm * tn + 7) / 8);
    gemm_nt_kernel<T, OutT><<<grid, 256, 0, s>>>(args, (OutT*)c, ldc, M, N, tm, tn);
}

template <typename T, typename OutT>
void launch_tn(const void* a, int lda, const void* b, int ldb, void* c, long ldc, int M, int N,
               int K, hipStream_t s) {
    const int tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
    const unsigned grid = 8u * (unsigned)((tm * tn + 7) / 8);
    gemm_tn_kernel<T, OutT><<<grid, 256, 0, s>>>((const T*)a, lda, (const T*)b, ldb, (OutT*)c,
                                                 ldc, M, N, K, tm, tn);
}

}  // namespace

template <typename T>
void launch_out_proj_bwd(const ProjProblem& p, const void* o_cat, const void* g, const void* w_o,
                         float* dw_o, void* do_cat, hipStream_t s) {
    // dW_O [H dv, d_model] = O_cat^T G: TN with K = T tokens
    launch_tn<T, float>(o_cat, p.hdv, g, p.d_model, dw_o, p.d_model, p.hdv, p.d_model, p.T, s);
    // dO_cat [T, H dv] = G W_O^T: NT with K = d_model (W_O rows are the N index)
    NTArgs a{};
    a.a[0] = g;
    a.b[0] = w_o;
    a.k[0] = p.d_model;
    a.lda[0] = p.d_model;
    a.ldb[0] = p.d_model;
    a.count = 1;
    launch_nt<T, T>(a, do_cat, p.hdv, p.T, p.hdv, s);
}

template <typename T>
void launch_in_proj_bwd(const ProjProblem& p, const void* x, const void* w_q, const void* w_k,
                        const void* w_v, const void* dq_cat, const void* dk_cat,
                        const void* dv_cat, float* dw_q, float* dw_k, float* dw_v, void* dx,
                        hipStream_t s) {
    // dW_P [d_model, H d_P] = X^T dP_cat: TN with K = T tokens
    launch_tn<T, float>(x, p.d_model, dq_cat, p.hd, dw_q, p.hd, p.d_model, p.hd, p.T, s);
    launch_tn<T, float>(x, p.d_model, dk_cat, p.hd, dw_k, p.hd, p.d_model, p.hd, p.T, s);
    launch_tn<T, float>(x, p.d_model, dv_cat, p.hdv, dw_v, p.hdv, p.d_model, p.hdv, p.T, s);
    // dX [T, d_model] = sum_P dP_cat W_P^T: NT, three products, K = H d_P
    NTArgs a{};
    const void* as[3] = {dq_cat, dk_cat, dv_cat};
    const void* bs[3] = {w_q, w_k, w_v};
    const int ks[3] = {p.hd, p.hd, p.hdv};
    for (int i = 0; i < 3; ++i) {
        a.a[i] = as[i];
        a.b[i] = bs[i];
        a.k[i] = ks[i];
        a.lda[i] = ks[i];
        a.ldb[i] = ks[i];
    }
    a.count = 3;
    launch_nt<T, T>(a, dx, p.d_model, p.T, p.d_model, s);
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template void launch_out_proj_bwd<ATTN_ELEM>(const ProjProblem&, const void*, const void*,
                                             const void*, float*, void*, hipStream_t);
template void launch_in_proj_bwd<ATTN_ELEM>(const ProjProblem&, const void*, const void*,
                                            const void*, const void*, const void*, const void*,
                                            const void*, float*, float*, float*, void*,
                                            hipStream_t);

}  // namespace attn

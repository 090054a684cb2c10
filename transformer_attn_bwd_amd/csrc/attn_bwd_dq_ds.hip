// dQ of backward attention from stored dS tiles (the stored-dS dQ mode).
//
// dQ_i = scale * sum_j dS_ij K_j (eulerpad "Attention backward" P5;
// mlgrind "Backward"), where dS = P o (dP - D) was formed, rounded to the
// input type, by the dK/dV kernel and written to the workspace as tiles of
// 256 keys x 256 queries, blocks of [256 keys][32 queries] row-major
// (attn_launch.h, DsTiles).
// This pass recomputes nothing: it is the product dQ^T = K^T dS^T per
// head, one workgroup per 256 queries walking the key blocks their rows
// see.  Its MFMA work is a fifth of the backward's; its bytes are the dS
// tiles (2 bytes per visible query-key pair), so it is bound by HBM.
//
// Layout: four waves, wave w owning queries i0 + 64w .. +63 (two 32-query
// MFMA tiles).  Per 64-key step the K rows go to LDS for every wave and
// each wave's 64 x 64 block of dS^T to its own part of LDS, both by buffer
// loads straight into swizzled tiles, three LDS stages with the fills two
// steps ahead.  Both operands come out of LDS with transposing reads: K^T
// (rows = d, k = keys) and dS^T (k = keys, columns = queries) in the same
// row-of-C key order (attn_device.h), so their product is dQ^T.  Causal
// masking needs no work here: the stored dS is exactly zero above the
// diagonal.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

constexpr int kDqsWaves = 4;
constexpr int kDqsRows = 64 * kDqsWaves;   // queries per workgroup
constexpr int kDqsKeys = 64;               // keys per step

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_ds_kernel(
    const T* __restrict__ k, const T* __restrict__ dsw, T* __restrict__ dq, DsTiles dst, int n,
    int m, int dg, float scale, int causal, SeqInfo si) {
    constexpr int BN = kDqsKeys, NW = kDqsWaves;
    // Three stages of (K tile, four waves' dS^T blocks): 3 x (16 + 32) KB at
    // d = 128.  The epilogue stages its rows in sS0.
    __shared__ __align__(1024) T sK0[BN * D];
    __shared__ __align__(1024) T sK1[BN * D];
    __shared__ __align__(1024) T sK2[BN * D];
    __shared__ __align__(1024) T sS0[NW * BN * 64];
    __shared__ __align__(1024) T sS1[NW * BN * 64];
    __shared__ __align__(1024) T sS2[NW * BN * 64];
    auto Kbuf = [&](auto b_) __attribute__((always_inline)) -> T* {
        constexpr int b = decltype(b_)::value;
        if constexpr (b == 0) return sK0;
        else if constexpr (b == 1) return sK1;
        else return sK2;
    };
    auto Sbuf = [&](auto b_) __attribute__((always_inline)) -> T* {
        constexpr int b = decltype(b_)::value;
        if constexpr (b == 0) return sS0;
        else if constexpr (b == 1) return sS1;
        else return sS2;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const TileOrder to = tile_order((int)gridDim.x, (int)gridDim.y);
    const long bh = to.head;
    const int qb = causal ? (int)gridDim.y - 1 - to.rank : to.rank;
    const int i0 = qb * kDqsRows;
    const SeqLens len = seq_lens(si, bh, n, m);
    const int nb = len.n, mb = len.m;
    const HeadView hk = head_view(si, bh, m, dg), hq = head_view(si, bh, n, dg);

    // Keys this block's rows see: all mb, or under the causal mask those up
    // to its last row.  The tiles of key blocks beyond were never written.
    int k_end = causal ? min(mb, i0 + kDqsRows) : mb;
    if (i0 >= nb) k_end = 0;
    const int nsteps = (max(k_end, 0) + BN - 1) / BN;

    const __amdgpu_buffer_rsrc_t rK = make_rsrc(k + hk.base, (uint32_t)mb * hk.stride * 2);
    const __amdgpu_buffer_rsrc_t rS =
        make_rsrc(dsw + bh * dst.head_elems, (uint32_t)(dst.head_elems * 2));
    TileLoader<D, BN, NW> ldK;
    ldK.init(wave, lane, dg, hk.stride);
    // This wave's 64 x 64 block of dS^T (keys x queries) in LDS as a
    // swizzled SwzTile<64>: 16-byte chunk c of key row r comes from the
    // 32-query block c / 4 of the wave's two, row r, queries 8 (c % 4) ..
    // (element offsets from the first of the two blocks).
    constexpr int kSBlock = kDsTile * 32;   // elements per [256 keys][32 queries] block
    constexpr int kSLoads = BN * 8 / 64;    // 1 KB loads per wave
    int soff[kSLoads];
#pragma unroll
    for (int jj = 0; jj < kSLoads; ++jj) {
        const int p = jj * 64 + lane, r = p / 8, c = (p % 8) ^ SwzTile<64>::swz(r);
        soff[jj] = (c / 4) * kSBlock + r * 32 + 8 * (c % 4);
    }
    constexpr int kLoads = TileLoader<D, BN, NW>::N + kSLoads;

    // Step s: keys k0 = 64 s of key block r = k0 / 256: rows k0 % 256 .. +63
    // of this wave's two 32-query blocks (2 wave, 2 wave + 1) of tile (qb, r).
    auto stage = [&](auto b_, int s) __attribute__((always_inline)) {
        const int k0 = s * BN, r = k0 / kDsTile;
        tile_fill<D, BN, NW>(ldK, Kbuf(b_), rK, k0, wave);
        const long tile = dst.tri ? (long)qb * (qb + 1) / 2 + r : (long)qb * dst.mblk + r;
        const uint32_t so = (uint32_t)((tile * kDsTile * kDsTile + (long)(2 * wave) * kSBlock +
                                        (long)(k0 % kDsTile) * 32) * 2);
        T* dstl = Sbuf(b_) + wave * BN * 64;
#pragma unroll
        for (int jj = 0; jj < kSLoads; ++jj)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (ATTN_LDS void*)(dstl + jj * 512), 16,
                                                     (unsigned)(2 * soff[jj]), so, 0, 0);
    };

    TileOffsets<D> toK;
    toK.init(lane);
    TileOffsets<64> toS;
    toS.init(lane);

    f32x16 acc[D / 32][2];
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
        acc[x][0] = zero16();
        acc[x][1] = zero16();
    }

    // dQ^T[x][t] += K^T (d block x, keys of chunk c) dS^T (keys of chunk c,
    // query tile t), for the four 16-key chunks of the step.
    auto compute = [&](auto b_) __attribute__((always_inline)) {
        const T* Ks = Kbuf(b_);
        const T* Ss = Sbuf(b_) + wave * BN * 64;
#pragma unroll
        for (int c = 0; c < BN / 16; ++c) {
            vec8<T> bS[2], aK[D / 32];
#pragma unroll
            for (int t = 0; t < 2; ++t) bS[t] = tile_read_tr_at<64>(Ss, toS, 16 * c, t);
#pragma unroll
            for (int x = 0; x < D / 32; ++x) aK[x] = tile_read_tr_at<D>(Ks, toK, 16 * c, x);
#pragma unroll
            for (int x = 0; x < D / 32; ++x) {
                acc[x][0] = mfma32(aK[x], bS[0], acc[x][0]);
                acc[x][1] = mfma32(aK[x], bS[1], acc[x][1]);
            }
        }
    };

    // Fills run two steps ahead: step s waits for its own fill (the next
    // one, kLoads loads per wave, may stay in flight), then the barrier
    // makes every wave's part visible and frees buffer (s + 2) % 3, whose
    // last reader was step s - 1.
    auto do_step = [&](auto b_, int s) __attribute__((always_inline)) {
        constexpr int b = decltype(b_)::value;
        if (s + 1 < nsteps)
            __builtin_amdgcn_s_waitcnt(kLoads | 0x70 | 0xF00);   // vmcnt(kLoads)
        else
            __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);            // vmcnt(0)
        __syncthreads();
        if (s + 2 < nsteps) stage(std::integral_constant<int, (b + 2) % 3>{}, s + 2);
        compute(b_);
    };
    static_assert(kLoads < 16, "vmcnt immediate holds 4 bits here");

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    if (nsteps > 0) stage(B0{}, 0);
    if (nsteps > 1) stage(B1{}, 1);
    int s = 0;
    for (; s + 2 < nsteps; s += 3) {
        do_step(B0{}, s);
        do_step(B1{}, s + 1);
        do_step(B2{}, s + 2);
    }
    if (s < nsteps) do_step(B0{}, s);
    if (s + 1 < nsteps) do_step(B1{}, s + 1);
    __syncthreads();   // every wave is done with the buffers the epilogue reuses

    // Accumulator slot vv of tile (x, t) holds column d = 32x + 8(vv>>2) +
    // 4g + (vv&3) of query i0 + 64 wave + 32 t + li.  Rows at or past nb are
    // written as zeros (selected: their dS columns past the dK/dV kernel's
    // last query tile were never written).  The tiles go out through this
    // wave's 64 x 64 staging block: written row-major (16-byte chunks
    // XOR-swizzled by row), read back as whole rows and stored 16 bytes per
    // lane.
    T* reg = sS0 + wave * 64 * 64;
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc(dq + hq.base, (uint32_t)(n * hq.stride * 2));
    const int qw0 = i0 + 64 * wave;
#pragma unroll
    for (int sl = 0; sl < D / 64; ++sl) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = 32 * t + li;
            const bool real = qw0 + row < nb;
#pragma unroll
            for (int xs = 0; xs < 2; ++xs) {
#pragma unroll
                for (int vq = 0; vq < 4; ++vq) {
                    vec4<T> w;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        w[r] = (T)(acc[2 * sl + xs][t][4 * vq + r] * scale);
                    u32x2 bits = __builtin_bit_cast(u32x2, w);
                    bits = real ? bits : u32x2{0u, 0u};
                    const int chunk = 4 * xs + vq;
                    *reinterpret_cast<u32x2*>(reg + row * 64 + 8 * (chunk ^ (row & 7)) + 4 * g) = bits;
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
            const int col = 64 * sl + 8 * chunk;
            const uint32_t byte_off =
                col < dg ? (uint32_t)(((long)(qw0 + row) * hq.stride + col) * 2) : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w8[i]), rdq,
                                                   byte_off, 0, 0);
        }
    }
}

template <typename T, int D>
void launch_dqs(const Problem& p, const void* k, const Workspace& w, void* dq, hipStream_t s) {
    dim3 grid((unsigned)p.heads(), (unsigned)((p.n + kDqsRows - 1) / kDqsRows));
    bwd_dq_ds_kernel<T, D><<<grid, 64 * kDqsWaves, 0, s>>>(
        (const T*)k, (const T*)w.ds.p, (T*)dq, w.ds, p.n, p.m, p.d, p.scale, p.causal ? 1 : 0,
        seq_info(p));
}

}  // namespace

template <typename T>
bool launch_bwd_dq_ds_mfma(const Problem& p, const void* k, const Workspace& w, void* dq,
                           hipStream_t s) {
    switch (mfma_widths(p) >> 8) {
    case 0x40: launch_dqs<T, 64>(p, k, w, dq, s); break;
    case 0x80: launch_dqs<T, 128>(p, k, w, dq, s); break;
    default: return false;
    }
    return true;
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template bool launch_bwd_dq_ds_mfma<ATTN_ELEM>(const Problem&, const void*, const Workspace&,
                                              void*, hipStream_t);

}  // namespace attn

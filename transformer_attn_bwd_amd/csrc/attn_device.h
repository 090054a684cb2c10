// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the 32x32x16 bf16 MFMA, bf16 packing and the operand
// layouts the kernels rely on.
//
// MFMA v_mfma_f32_32x32x16_bf16, one wave of 64 lanes, lane l, g = l >> 5,
// li = l & 31:
//   A (32 x 16, M x K): lane l holds row li, eight k values in slots s=0..7
//   B (16 x 32, K x N): lane l holds column li, eight k values in slots s
//   C (32 x 32, M x N): lane l holds column li, rows 8*(v>>2) + 4*g + (v&3)
//                       in accumulator slots v = 0..15
// A and B place a given k at the same (g, s) position, so any assignment of
// logical k values to (g, s) gives the same product as long as both
// operands use it.  Two assignments are used:
//   natural:   k = 8*g + s                 (operands read from memory)
//   row-of-C:  k = 8*(s>>2) + 4*g + (s&3)  within a 16-row half c of a C
//              tile, i.e. C slots v = 8*c + s reused as an operand.  The
//              partner operand then reads rows 4g..4g+3 and 8+4g..8+4g+3,
//              two runs of four, which is what read_rowc_pair() fetches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Calls f(std::integral_constant<int, I>{}) for I = 0..N-1, so that every
// index inside f is a compile-time constant (register arrays stay arrays).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(static_cast<F&&>(f), std::make_integer_sequence<int, N>{});
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with the accumulator pinned in AGPRs, for kernels whose
// accumulators do not fit next to their other operands in the 256 VGPRs.
// Written out because the compiler places all MFMA results in one register
// file.  The compiler does not see this as an MFMA, so the hazards it
// would cover are covered here: s_nop 1 gives the two wait states an MFMA
// needs after a VALU write of its A or B operand; the accumulator is only
// ever touched by this chain, and callers wait (s_nop) before reading it.
__device__ __forceinline__ void mfma32_agpr(bf16x8 a, bf16x8 b, f32x16& acc) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Eight fp32 values -> eight bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
    r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
    return r;
}

// Accumulator slots 8c..8c+7 of a C tile as a bf16 operand (row-of-C order).
__device__ __forceinline__ bf16x8 c_half_to_bf16(const f32x16& x, int c) {
    return pack8(x[8 * c + 0], x[8 * c + 1], x[8 * c + 2], x[8 * c + 3],
                 x[8 * c + 4], x[8 * c + 5], x[8 * c + 6], x[8 * c + 7]);
}

// The partner of a row-of-C operand, from a transposed LDS tile whose row
// `p` (pointer to its first element) lists the C-tile rows contiguously:
// elements base+4g..base+4g+3 and base+8+4g..base+8+4g+3.
__device__ __forceinline__ bf16x8 read_rowc_pair(const bf16* p, int base, int g) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + base + 4 * g);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + base + 8 + 4 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 gload_bf16x8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ u32x4 gload16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void lds_write16(bf16* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ void lds_write8(bf16* p, u32x2 v) {
    *reinterpret_cast<u32x2*>(p) = v;
}

// Given four rows of eight bf16 (one 16-byte chunk each, rows r..r+3 of a
// tile, columns c..c+7), form column c+y of those four rows as four bf16
// packed in 8 bytes: the transposed piece written to a [col][row] LDS tile.
__device__ __forceinline__ u32x2 column4(const u32x4 (&rows)[4], int y) {
    const int w = y >> 1;
    u32x2 r;
    if (y & 1) {
        r[0] = (rows[0][w] >> 16) | (rows[1][w] & 0xffff0000u);
        r[1] = (rows[2][w] >> 16) | (rows[3][w] & 0xffff0000u);
    } else {
        r[0] = (rows[0][w] & 0xffffu) | (rows[1][w] << 16);
        r[1] = (rows[2][w] & 0xffffu) | (rows[3][w] << 16);
    }
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define ATTN_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// Swizzled row-major LDS tiles filled straight from global memory.
//
// A tile of ROWS x C bf16 is stored row-major in 16-byte chunks; chunk c of
// row r sits in slot c ^ swz(r).  The swizzle makes both access patterns the
// kernels use free of bank conflicts (64 banks x 4 bytes):
//  - operand reads of 16 bytes by 16 lanes on 16 consecutive rows, same chunk;
//  - transposing reads of 8 bytes by 32 lanes on 4 rows x 4 chunks.
// Tiles are written with global_load_lds_dwordx4: one wave instruction moves
// 1 KB, lane L filling the L-th 16-byte slot of that kilobyte, so the
// swizzle is applied on the global side by choosing which chunk each lane
// fetches.
template <int C>
struct SwzTile {
    static constexpr int CPR = C / 8;                    // 16-byte chunks per row
    static_assert(CPR == 8 || CPR == 16, "tile widths of 64 or 128 bf16");
    __device__ static __forceinline__ int swz(int r) {
        if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
        else return (((r >> 1) & 1) << 2) ^ ((r >> 2) & 3);
    }
    // element offset of chunk c (8 bf16) of row r
    __device__ static __forceinline__ int off(int r, int c) { return r * C + 8 * (c ^ swz(r)); }
};

// Per-lane element offsets into a swizzled C-wide tile for the two read
// patterns the kernels use.  Row-block parts that are multiples of 16 rows
// (query or key halves, 16-row halves of a C tile) do not change the
// swizzle, so they are left to the instructions' immediate offsets.
//  a[kc]:      operand read of row (lane & 31), chunk 2*kc + (lane >> 5)
//  tr[h][nt]:  transposing read of rows 4g + (j>>2) + 8h (g = lane>>5,
//              j = lane & 15), columns 32*nt + 16*((lane>>4)&1) + 4*(j&3)
template <int C>
struct TileOffsets {
    int a[C / 16];
    int tr[2][C / 32];
    __device__ __forceinline__ void init(int lane) {
        using T = SwzTile<C>;
        const int li = lane & 31, g = lane >> 5;
#pragma unroll
        for (int kc = 0; kc < C / 16; ++kc) a[kc] = T::off(li, 2 * kc + g);
        const int blk = lane >> 4, j = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 4 * g + (j >> 2) + 8 * h;
#pragma unroll
            for (int nt = 0; nt < C / 32; ++nt) {
                const int col = 32 * nt + 16 * (blk & 1) + 4 * (j & 3);
                tr[h][nt] = T::off(r, col >> 3) + (col & 7);
            }
        }
    }
};

// Operand read through precomputed offsets: rows row0 + (lane & 31) of a
// tile at `tile` (row0 a multiple of 16), chunk 2*kc + g.
template <int C>
__device__ __forceinline__ bf16x8 tile_read8_at(const bf16* tile, const TileOffsets<C>& to,
                                                int row0, int kc) {
    return *reinterpret_cast<const bf16x8*>(tile + row0 * C + to.a[kc]);
}

// Transposing read through precomputed offsets; `base` (a multiple of 16)
// is the first of the 16 tile rows that form the k range, nt the 32-column
// block: lane l gets column 32*nt + (l & 31) of rows base+4g..+3 and
// base+8+4g..+3.
template <int C>
__device__ __forceinline__ bf16x8 tile_read_tr_at(const bf16* tile, const TileOffsets<C>& to,
                                                  int base, int nt) {
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (ATTN_LDS i16x4*)(tile + base * C + to.tr[0][nt]));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (ATTN_LDS i16x4*)(tile + base * C + to.tr[1][nt]));
    i16x4 both[2] = {lo, hi};
    return *reinterpret_cast<bf16x8*>(both);
}

// Fill ROWS rows of a swizzled tile from global rows row0.. of a [*, C]
// row-major bf16 matrix, the work split over NW waves (this is wave w);
// rows at or past `valid` read row valid-1 instead (callers neutralise
// them).
template <int C, int ROWS, int NW>
__device__ __forceinline__ void tile_load_split(bf16* lds_tile, const bf16* g, int row0,
                                                int valid, int w, int lane) {
    using T = SwzTile<C>;
    constexpr int INSTS = ROWS * T::CPR / 64;
    static_assert(INSTS % NW == 0, "tile loads must split evenly over the waves");
#pragma unroll
    for (int jj = 0; jj < INSTS / NW; ++jj) {
        const int ii = w + NW * jj;
        const int p = ii * 64 + lane;
        const int r = p / T::CPR;
        const int s = p % T::CPR;
        int grow = row0 + r;
        grow = grow < valid ? grow : valid - 1;
        const bf16* src = g + (long)grow * C + 8 * (s ^ T::swz(r));
        __builtin_amdgcn_global_load_lds(src, (ATTN_LDS void*)(lds_tile + ii * 512), 16, 0, 0);
    }
}

// The tile_load_split pattern with the per-lane source offsets computed
// once: load jj of wave w fills kilobyte ii = w + NW*jj of the tile, this
// lane fetching chunk s ^ swz(r) of tile row r (p = 64 ii + lane, r = p /
// CPR, s = p % CPR); off[jj] is that chunk's element offset from the
// tile's first global row.
template <int C, int ROWS, int NW>
struct TileLoader {
    using T = SwzTile<C>;
    static constexpr int N = ROWS * T::CPR / 64 / NW;
    static_assert(N * 64 * NW == ROWS * T::CPR, "tile loads must split evenly over the waves");
    int off[N];
    __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
        for (int jj = 0; jj < N; ++jj) {
            const int p = (w + NW * jj) * 64 + lane;
            const int r = p / T::CPR, s = p % T::CPR;
            off[jj] = r * C + 8 * (s ^ T::swz(r));
        }
    }
};

// Buffer resource for a raw byte range [base, base + bytes): loads through
// it at offsets past the end return zeros (the fourth descriptor word
// selects 32-bit raw data, the usual value for untyped buffer access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Fill a tile from rows row0 .. row0 + ROWS - 1 of the [*, C] bf16 matrix
// behind `rsrc` (buffer loads straight into LDS); rows past the end of the
// buffer come back as zeros.
template <int C, int ROWS, int NW>
__device__ __forceinline__ void tile_fill(const TileLoader<C, ROWS, NW>& L, bf16* lds_tile,
                                          __amdgpu_buffer_rsrc_t rsrc, int row0, int w) {
#pragma unroll
    for (int jj = 0; jj < TileLoader<C, ROWS, NW>::N; ++jj)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(lds_tile + (w + NW * jj) * 512),
                                                 16, (unsigned)(2 * L.off[jj]),
                                                 (unsigned)(2 * row0 * C), 0, 0);
}

// One of the INSTS/NW loads tile_load_split would issue (number jj), so
// that a tile's loads can be spread over a step instead of issued at once.
template <int C, int ROWS, int NW>
__device__ __forceinline__ void tile_load_one(bf16* lds_tile, const bf16* g, int row0, int valid,
                                              int w, int lane, int jj) {
    using T = SwzTile<C>;
    const int ii = w + NW * jj;
    const int p = ii * 64 + lane;
    const int r = p / T::CPR;
    const int s = p % T::CPR;
    int grow = row0 + r;
    grow = grow < valid ? grow : valid - 1;
    const bf16* src = g + (long)grow * C + 8 * (s ^ T::swz(r));
    __builtin_amdgcn_global_load_lds(src, (ATTN_LDS void*)(lds_tile + ii * 512), 16, 0, 0);
}
template <int C, int ROWS, int NW>
constexpr int tile_loads_per_wave() { return ROWS * (C / 8) / 64 / NW; }

// Fill `rows` rows of a swizzled tile from global rows row0.. of a [*, C]
// row-major bf16 matrix; rows at or past `valid` read row valid-1 instead
// (callers neutralise them).  Called by `nw` waves, wave `w`.
template <int C, int ROWS>
__device__ __forceinline__ void tile_load_async(bf16* lds_tile, const bf16* g, int row0,
                                                int valid, int w, int nw, int lane) {
    using T = SwzTile<C>;
    constexpr int INSTS = ROWS * T::CPR / 64;
    for (int ii = w; ii < INSTS; ii += nw) {
        const int p = ii * 64 + lane;
        const int r = p / T::CPR;
        const int s = p % T::CPR;
        int grow = row0 + r;
        grow = grow < valid ? grow : valid - 1;
        const bf16* src = g + (long)grow * C + 8 * (s ^ T::swz(r));
        __builtin_amdgcn_global_load_lds(src, (ATTN_LDS void*)(lds_tile + ii * 512), 16, 0, 0);
    }
}

// 8 contiguous bf16 of row r, chunk c (an MFMA operand in natural k order).
template <int C>
__device__ __forceinline__ bf16x8 tile_read8(const bf16* lds_tile, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(lds_tile + SwzTile<C>::off(r, c));
}

// Transposing read: the partner of a row-of-C operand.  Lane l (g = l>>5)
// receives column n0 + (l & 31) of rows base+4g..base+4g+3 (slots 0-3) and
// base+8+4g..base+8+4g+3 (slots 4-7), from a swizzled row-major tile.
// ds_read_b64_tr_b16 works on blocks of 16 lanes: lane i of a block gets
// element (i & 3) of the 8-byte rows addressed by lanes 4e+(i>>2), e=0..3.
template <int C>
__device__ __forceinline__ bf16x8 tile_read_tr(const bf16* lds_tile, int base, int n0, int lane) {
    const int blk = lane >> 4, j = lane & 15;
    const int g = blk >> 1;
    const int col = n0 + 16 * (blk & 1) + 4 * (j & 3);
    const int r = base + 4 * g + (j >> 2);
    const int o0 = SwzTile<C>::off(r, col >> 3) + (col & 7);
    const int o1 = SwzTile<C>::off(r + 8, col >> 3) + (col & 7);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(lds_tile + o0));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(lds_tile + o1));
    i16x4 both[2] = {lo, hi};
    return *reinterpret_cast<bf16x8*>(both);
}

__device__ __forceinline__ float xor_lane32(float x) {
    // exchange with the lane 32 positions away (the other half of the wave)
    return __shfl_xor(x, 32, 64);
}

}  // namespace attn

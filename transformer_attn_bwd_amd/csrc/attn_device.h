// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the 32x32x16 MFMAs on 16-bit inputs (bfloat16 and IEEE
// half, float32 accumulation), packing to 16 bits and the operand layouts
// the kernels rely on.  Kernels are written once over the element type T
// (bf16 or f16); only the MFMA opcode and the float -> T rounding differ.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16}, one wave of 64 lanes, lane l,
// g = l >> 5, li = l & 31:
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
//              two runs of four, which is what the transposing LDS read
//              (tile_read_tr_at) fetches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn {

typedef __bf16 bf16;
typedef _Float16 f16;
template <typename T>
using vec8 = T __attribute__((ext_vector_type(8)));
template <typename T>
using vec4 = T __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ f32x16 mfma32(vec8<bf16> a, vec8<bf16> b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(vec8<f16> a, vec8<f16> b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The same products with the accumulator pinned in AGPRs, for kernels whose
// accumulators do not fit next to their other operands in the 256 VGPRs.
// Written out because the compiler places all MFMA results in one register
// file.  The compiler does not see these as MFMAs, so it inserts none of
// the wait states an MFMA needs around it: the two after a VALU write of
// its A or B operand, given here by an s_nop 1 unless the caller's schedule
// keeps such writes two instructions away by itself (WAIT = false, used
// where the build's hazard check finds it so in the assembly; it fails the
// build otherwise), and the 18 before anything else reads the accumulator
// (callers end the chain with mfma_agpr_wait and mfma_agpr_fence).
template <bool WAIT = true>
__device__ __forceinline__ void mfma32_agpr(vec8<bf16> a, vec8<bf16> b, f32x16& acc) {
    if constexpr (WAIT)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool WAIT = true>
__device__ __forceinline__ void mfma32_agpr(vec8<f16> a, vec8<f16> b, f32x16& acc) {
    if constexpr (WAIT)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last mfma32_agpr writing an accumulator and any
// other read of it (24, more than the 18 a 32x32 MFMA result needs before a
// VALU or v_accvgpr_read reads it).  A wait alone is not enough: the
// compiler may schedule a register move of an accumulator (v_accvgpr_read)
// anywhere after the last asm statement that names it, before the wait,
// where it reads a value the MFMA has not written yet.  So each
// accumulator passes through an asm statement placed after the wait
// (volatile asm statements keep their order), and every read of it comes
// after that.
__device__ __forceinline__ void mfma_agpr_wait() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
__device__ __forceinline__ void mfma_agpr_fence(f32x16& acc) { asm volatile("" : "+a"(acc)); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Eight fp32 values -> eight T (round to nearest even).
template <typename T>
__device__ __forceinline__ vec8<T> pack8(float a0, float a1, float a2, float a3, float a4,
                                         float a5, float a6, float a7) {
    vec8<T> r;
    r[0] = (T)a0; r[1] = (T)a1; r[2] = (T)a2; r[3] = (T)a3;
    r[4] = (T)a4; r[5] = (T)a5; r[6] = (T)a6; r[7] = (T)a7;
    return r;
}

// Sixteen bytes of global memory as eight T.
template <typename T>
__device__ __forceinline__ vec8<T> gload8(const T* p) {
    return *reinterpret_cast<const vec8<T>*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define ATTN_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// Swizzled row-major LDS tiles filled straight from global memory.
//
// A tile of ROWS x C 16-bit elements is stored row-major in 16-byte
// chunks; chunk c of row r sits in slot c ^ swz(r).  The swizzle makes both access patterns the
// kernels use free of bank conflicts (64 banks x 4 bytes):
//  - operand reads of 16 bytes by 16 lanes on 16 consecutive rows, same chunk;
//  - transposing reads of 8 bytes by 32 lanes on 4 rows x 4 chunks.
// Tiles are written with 16-byte buffer loads straight to LDS: one wave
// instruction moves 1 KB, lane L filling the L-th 16-byte slot of that
// kilobyte, so the swizzle is applied on the global side by choosing which
// chunk each lane fetches.
template <int C>
struct SwzTile {
    static constexpr int CPR = C / 8;                    // 16-byte chunks per row
    static_assert(CPR == 8 || CPR == 16, "tile widths of 64 or 128 elements");
    __device__ static __forceinline__ int swz(int r) {
        if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
        else return (((r >> 1) & 1) << 2) ^ ((r >> 2) & 3);
    }
    // element offset of chunk c (8 elements) of row r
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
template <int C, typename T>
__device__ __forceinline__ vec8<T> tile_read8_at(const T* tile, const TileOffsets<C>& to,
                                                 int row0, int kc) {
    return *reinterpret_cast<const vec8<T>*>(tile + row0 * C + to.a[kc]);
}

// Transposing read through precomputed offsets; `base` (a multiple of 16)
// is the first of the 16 tile rows that form the k range, nt the 32-column
// block: lane l gets column 32*nt + (l & 31) of rows base+4g..+3 and
// base+8+4g..+3.
template <int C, typename T>
__device__ __forceinline__ vec8<T> tile_read_tr_at(const T* tile, const TileOffsets<C>& to,
                                                   int base, int nt) {
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (ATTN_LDS i16x4*)(tile + base * C + to.tr[0][nt]));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (ATTN_LDS i16x4*)(tile + base * C + to.tr[1][nt]));
    i16x4 both[2] = {lo, hi};
    return *reinterpret_cast<vec8<T>*>(both);
}

// Element offset that lies past the end of every buffer the kernels read
// (the C ABI keeps each head's byte range within 2^30): a buffer load there
// returns zeros.
constexpr int kPastEnd = 0x3ff00000;

// Per-lane source offsets for filling a ROWS x C tile with NW waves from a
// matrix whose rows hold `width` <= C elements (a multiple of 8) and start
// `stride` elements apart, computed once: load jj of wave w fills kilobyte
// ii = w + NW*jj of the tile, this lane fetching chunk c = s ^ swz(r) of
// tile row r (p = 64 ii + lane, r = p / CPR, s = p % CPR); off[jj] is that
// chunk's element offset from the tile's first global row, or kPastEnd for
// chunks c >= width/8, which then fill with zeros (a narrower head is
// padded to the tile width).
template <int C, int ROWS, int NW>
struct TileLoader {
    using T = SwzTile<C>;
    static constexpr int N = ROWS * T::CPR / 64 / NW;
    static_assert(N * 64 * NW == ROWS * T::CPR, "tile loads must split evenly over the waves");
    int off[N];
    int stride;   // elements from one global row to the next
    __device__ __forceinline__ void init(int w, int lane, int width = C, int row_stride = 0) {
        stride = row_stride > 0 ? row_stride : width;
#pragma unroll
        for (int jj = 0; jj < N; ++jj) {
            const int p = (w + NW * jj) * 64 + lane;
            const int r = p / T::CPR, c = (p % T::CPR) ^ T::swz(r);
            off[jj] = 8 * c < width ? r * stride + 8 * c : kPastEnd;
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

// Fill a tile from rows row0 .. row0 + ROWS - 1 of the T matrix behind
// `rsrc` (buffer loads straight into LDS); rows past the end of the
// buffer, and columns width .. C-1, come back as zeros.
template <int C, int ROWS, int NW, typename T>
__device__ __forceinline__ void tile_fill(const TileLoader<C, ROWS, NW>& L, T* lds_tile,
                                          __amdgpu_buffer_rsrc_t rsrc, int row0, int w) {
#pragma unroll
    for (int jj = 0; jj < TileLoader<C, ROWS, NW>::N; ++jj)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (ATTN_LDS void*)(lds_tile + (w + NW * jj) * 512),
                                                 16, (unsigned)(2 * L.off[jj]),
                                                 (unsigned)(2 * row0 * L.stride), 0, 0);
}

__device__ __forceinline__ float xor_lane32(float x) {
    // exchange with the lane 32 positions away (the other half of the wave)
    return __shfl_xor(x, 32, 64);
}

}  // namespace attn

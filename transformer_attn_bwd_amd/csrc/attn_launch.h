// Internal interface between the C ABI (attn_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

// Element types, the values of enum attn_dtype in attn.h.
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kDtypeF16 = 2;

struct Problem {
    long B = 0, H = 0;
    int n = 0, m = 0, d = 0, dv = 0;
    float scale = 1.f;
    bool causal = false;
    int dtype = 0;
    long heads() const { return B * H; }
};

// Rows per head in the backward workspace (per-row D and rescaled LSE),
// padded so that every query tile the kernels touch is in bounds.
constexpr int kRowPad = 128;
inline int padded_rows(int n) { return (n + kRowPad - 1) / kRowPad * kRowPad; }

// Workspace view: lse2 [B*H][n_pad] then D [B*H][n_pad], float32.
struct Workspace {
    float* lse2;
    float* D;
    int n_pad;
};

// 16-bit MFMA path (p.dtype kDtypeBF16 or kDtypeF16); return false if
// (d, dv) or the dtype has no instantiation.
bool launch_fwd_mfma(const Problem& p, const void* q, const void* k, const void* v, void* o,
                     float* lse, hipStream_t s);
bool launch_bwd_preprocess_mfma(const Problem& p, const void* o, const void* dout,
                                const float* lse, const Workspace& w, hipStream_t s);
bool launch_bwd_dkdv_mfma(const Problem& p, const void* q, const void* k, const void* v,
                          const void* dout, const Workspace& w, void* dk, void* dv,
                          hipStream_t s);
bool launch_bwd_dq_mfma(const Problem& p, const void* q, const void* k, const void* v,
                        const void* dout, const Workspace& w, void* dq, hipStream_t s);

// fp32 path (one wave per row; any d, dv in 1..128).
bool launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o,
                    float* lse, hipStream_t s);
bool launch_bwd_preprocess_f32(const Problem& p, const float* o, const float* dout,
                               const float* lse, const Workspace& w, hipStream_t s);
bool launch_bwd_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v,
                         const float* dout, const Workspace& w, float* dk, float* dv,
                         hipStream_t s);
bool launch_bwd_dq_f32(const Problem& p, const float* q, const float* k, const float* v,
                       const float* dout, const Workspace& w, float* dq, hipStream_t s);

}  // namespace attn

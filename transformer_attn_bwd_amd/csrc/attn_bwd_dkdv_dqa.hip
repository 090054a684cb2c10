// The dK/dV kernel with the fused dQ contribution (attn_bwd_dkdv.h): the
// workgroups whose first key is at or past dqa_from also add dS K for their
// keys to the float32 dQ accumulator with atomics; the others run exactly
// as the plain kernel.
#include "attn_bwd_dkdv.h"

namespace attn {

template <typename T>
bool launch_bwd_dkdv_dqa_mfma(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dout, const Workspace& w, void* dk, void* dv,
                              float* dqacc, int dqa_from, hipStream_t s) {
    switch (mfma_widths(p)) {
    case 0x4040: launch_dkdv<T, 64, 64, true>(p, q, k, v, dout, w, dk, dv, dqacc, dqa_from, s); break;
    case 0x4080: launch_dkdv<T, 64, 128, true>(p, q, k, v, dout, w, dk, dv, dqacc, dqa_from, s); break;
    case 0x8040: launch_dkdv<T, 128, 64, true>(p, q, k, v, dout, w, dk, dv, dqacc, dqa_from, s); break;
    case 0x8080: launch_dkdv<T, 128, 128, true>(p, q, k, v, dout, w, dk, dv, dqacc, dqa_from, s); break;
    default: return false;
    }
    return true;
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template bool launch_bwd_dkdv_dqa_mfma<ATTN_ELEM>(const Problem&, const void*, const void*,
                                                 const void*, const void*, const Workspace&,
                                                 void*, void*, float*, int, hipStream_t);

}  // namespace attn

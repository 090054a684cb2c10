// The dK/dV kernel of the stored-dS dQ mode (attn_bwd_dkdv.h with DSS):
// besides dK and dV, every workgroup writes the 16-bit dS it forms for its
// 256 keys, one 32-query step at a time, into the workspace's dS tiles,
// which the dQ = dS K pass (attn_bwd_dq_ds.hip) reads back.
#include "attn_bwd_dkdv.h"

namespace attn {

template <typename T>
bool launch_bwd_dkdv_dss_mfma(const Problem& p, const void* q, const void* k, const void* v,
                              const void* dout, const Workspace& w, void* dk, void* dv,
                              hipStream_t s) {
    switch (mfma_widths(p)) {
    case 0x4040: launch_dkdv<T, 64, 64, false, true>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    case 0x4080: launch_dkdv<T, 64, 128, false, true>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    case 0x8040: launch_dkdv<T, 128, 64, false, true>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    case 0x8080: launch_dkdv<T, 128, 128, false, true>(p, q, k, v, dout, w, dk, dv, nullptr, 0, s); break;
    default: return false;
    }
    return true;
}

// Each element type is compiled as its own object (-DATTN_ELEM=bf16 or f16)
// so that the builds of the two instantiations run in parallel.
#ifndef ATTN_ELEM
#error "compile once per element type: -DATTN_ELEM=bf16 or -DATTN_ELEM=f16"
#endif
template bool launch_bwd_dkdv_dss_mfma<ATTN_ELEM>(const Problem&, const void*, const void*,
                                                 const void*, const void*, const Workspace&,
                                                 void*, void*, hipStream_t);

}  // namespace attn

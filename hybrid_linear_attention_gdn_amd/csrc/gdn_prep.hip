// The intra-chunk preparation kernel with ordinary stores (one store kind per
// translation unit; see gdn_prep.h).

#include "gdn_prep.h"
#include "gdn_launch.h"

namespace gdn {

hipError_t launch_prep(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                       const int32_t* cu, int n_seqs, int h_qk, int h_v, const ChunkWorkspace& ws, int slot_lo,
                       int slot_hi, hipStream_t stream)
{
    if (prep_heads(h_qk, h_v) == 2)
        hipLaunchKernelGGL((gdn_chunk_prep<false, 2>), dim3(slots_x8(slot_hi - slot_lo), h_v / 2), dim3(256), 0, stream,
                           q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, slot_lo, slot_hi);
    else
        hipLaunchKernelGGL((gdn_chunk_prep<false, 1>), dim3(slots_x8(slot_hi - slot_lo), h_v), dim3(256), 0, stream,
                           q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, slot_lo, slot_hi);
    return hipGetLastError();
}

}  // namespace gdn

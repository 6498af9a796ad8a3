// The backward's state-recompute pass with reset flags for bf16 sequences: the
// forward kernel template in states-only mode with the backward's chunk length.
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_chunk_states_reset_bf16(const FwdParams& p, int disc, bool vec,
                                           hipStream_t stream) {
  return dispatch_fwd_reset_t<bf16_t, kItemsBwd, kModeChunkStates>(p, disc, vec, stream);
}

hipError_t dispatch_chunk_states_fix_reset_bf16(const FwdParams& p, int disc, bool vec,
                                            hipStream_t stream) {
  return dispatch_fwd_reset_t<bf16_t, kItemsBwd, kModeChunkStates, true>(p, disc, vec, stream);
}

}  // namespace mscan

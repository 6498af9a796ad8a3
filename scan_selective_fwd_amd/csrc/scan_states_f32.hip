// The backward's state-recompute pass for f32 sequences: the forward kernel
// template in states-only mode with the backward's chunk length.
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_chunk_states_f32(const FwdParams& p, int disc, int lanes, bool vec,
                                      hipStream_t stream) {
  return dispatch_fwd_t<float, kItemsBwd, kModeChunkStates>(p, disc, lanes, vec, stream);
}

hipError_t dispatch_chunk_states_fix_f32(const FwdParams& p, int disc, bool vec,
                                      hipStream_t stream) {
  return dispatch_fwd_fix_t<float, kItemsBwd, kModeChunkStates>(p, disc, vec, stream);
}

}  // namespace mscan

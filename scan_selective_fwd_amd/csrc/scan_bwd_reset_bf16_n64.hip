// Backward kernels for bf16 sequences with reset flags (packed sequences),
// N in 17..64 (see scan_bwd_impl.hpp).
#include "scan_bwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_bwd_reset_bf16_n64(const BwdParams& p, int disc, bool vec, hipStream_t stream,
                                            hipEvent_t ev_begin, hipEvent_t ev_end) {
  return dispatch_bwd_nt<bf16_t, 64, true>(p, disc, vec, stream, ev_begin, ev_end);
}

}  // namespace mscan

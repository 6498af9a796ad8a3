// Backward kernels for f32 sequences,
// N <= 16 (see scan_bwd_impl.hpp).
#include "scan_bwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_bwd_f32_n16(const BwdParams& p, int disc, bool vec, hipStream_t stream,
                                     hipEvent_t ev_begin, hipEvent_t ev_end) {
  return dispatch_bwd_nt<float, 16, false>(p, disc, vec, stream, ev_begin, ev_end);
}

}  // namespace mscan

// Forward-scan kernels with reset flags (packed sequences) for bf16 sequences
// (see scan_fwd_impl.hpp): the output pass and the segment summary pass.
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_fwd_reset_bf16(const FwdParams& p, int disc, bool vec, hipStream_t stream) {
  return dispatch_fwd_reset_t<bf16_t, kItems, kModeOut>(p, disc, vec, stream);
}

hipError_t dispatch_seg_summary_reset_bf16(const FwdParams& p, int disc, bool vec,
                                          hipStream_t stream) {
  return dispatch_fwd_reset_t<bf16_t, kItems, kModeSegSummary>(p, disc, vec, stream);
}

}  // namespace mscan

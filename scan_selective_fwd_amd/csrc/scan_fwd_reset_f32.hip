// Forward-scan kernels with reset flags (packed sequences) for f32 sequences
// (see scan_fwd_impl.hpp): the output pass, the summary pass and the
// correcting launch of a segmented run.
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_fwd_reset_f32(const FwdParams& p, int disc, bool vec, hipStream_t stream) {
  return dispatch_fwd_reset_t<float, kItems, kModeOut>(p, disc, vec, stream);
}

hipError_t dispatch_scan_fwd_fix_reset_f32(const FwdParams& p, int disc, bool vec,
                                          hipStream_t stream) {
  return dispatch_fwd_reset_t<float, kItems, kModeOut, true>(p, disc, vec, stream);
}

hipError_t dispatch_seg_summary_reset_f32(const FwdParams& p, int disc, bool vec,
                                          hipStream_t stream) {
  return disc == 0 ? fwd_nv<float, 16, kItems, true, kModeSegSummary, true>(p, vec, stream)
                   : fwd_nv<float, 16, kItems, false, kModeSegSummary, true>(p, vec, stream);
}

}  // namespace mscan

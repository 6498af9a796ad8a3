// Forward-scan kernels for f32 sequences (see scan_fwd_impl.hpp).
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_fwd_f32(const FwdParams& p, int disc, int lanes, bool vec,
                                  hipStream_t stream) {
  return dispatch_fwd_t<float, kItems, kModeOut>(p, disc, lanes, vec, stream);
}

hipError_t dispatch_scan_fwd_fix_f32(const FwdParams& p, int disc, bool vec, hipStream_t stream) {
  return dispatch_fwd_fix_t<float, kItems, kModeOut>(p, disc, vec, stream);
}

hipError_t dispatch_seg_summary_f32(const FwdParams& p, int disc, bool vec, hipStream_t stream) {
  return disc == 0 ? fwd_nv<float, 16, kItems, true, kModeSegSummary>(p, vec, stream)
                   : fwd_nv<float, 16, kItems, false, kModeSegSummary>(p, vec, stream);
}

}  // namespace mscan

// Forward-scan kernels for bf16 sequences (see scan_fwd_impl.hpp).
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_fwd_bf16(const FwdParams& p, int disc, int lanes, bool vec,
                                  hipStream_t stream) {
  return dispatch_fwd_t<bf16_t, kItems, kModeOut>(p, disc, lanes, vec, stream);
}

hipError_t dispatch_scan_fwd_fix_bf16(const FwdParams& p, int disc, bool vec, hipStream_t stream) {
  return dispatch_fwd_fix_t<bf16_t, kItems, kModeOut>(p, disc, vec, stream);
}

hipError_t dispatch_seg_summary_bf16(const FwdParams& p, int disc, bool vec, hipStream_t stream) {
  return disc == 0 ? fwd_nv<bf16_t, 16, kItems, true, kModeSegSummary>(p, vec, stream)
                   : fwd_nv<bf16_t, 16, kItems, false, kModeSegSummary>(p, vec, stream);
}

}  // namespace mscan

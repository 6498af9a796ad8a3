// Forward-scan kernels for f32 sequences (see scan_fwd_impl.hpp).
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_fwd_f32(const FwdParams& p, int disc, int lanes, bool vec,
                                  hipStream_t stream) {
  return dispatch_fwd_t<float, kItems, false>(p, disc, lanes, vec, stream);
}

}  // namespace mscan

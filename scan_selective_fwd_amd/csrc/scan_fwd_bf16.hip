// Forward-scan kernels for bf16 sequences (see scan_fwd_impl.hpp).
#include "scan_fwd_impl.hpp"

namespace mscan {

hipError_t dispatch_scan_fwd_bf16(const FwdParams& p, int disc, int lanes, bool vec,
                                  hipStream_t stream) {
  return dispatch_fwd_t<bf16_t, kItems, false>(p, disc, lanes, vec, stream);
}

}  // namespace mscan

// Host-only stand-ins for the kernel dispatchers.  With them the C ABI layer
// (api.cpp: argument checks, size, workspace and layout arithmetic) builds
// with the host compiler and runs under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Each stand-in
// counts that it was reached and launches nothing.
#include "kernels.hpp"

namespace mscan {

int g_dispatched = 0;

namespace {
hipError_t reached() {
  ++g_dispatched;
  return hipSuccess;
}
}  // namespace

hipError_t dispatch_scan_fwd_complex(const CplxParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_complex(const CplxParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_seg_summary_complex(const CplxParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_seg_carry_complex(const CplxParams&, hipStream_t) { return reached(); }
hipError_t dispatch_bwd_seg_summary_complex(const CplxBwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_bwd_seg_carry_complex(const CplxBwdParams&, hipStream_t) { return reached(); }
hipError_t dispatch_scan_bwd_complex(const CplxBwdParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_conv_fwd(const ConvParams&, int, bool, hipStream_t) { return reached(); }
hipError_t dispatch_conv_bwd(const ConvParams&, int, bool, hipStream_t) { return reached(); }
hipError_t dispatch_scan_fwd_f32(const FwdParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_bf16(const FwdParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_f32(const FwdParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_bf16(const FwdParams&, int, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_reset_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_reset_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_fix_reset_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_fix_reset_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_reset_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_reset_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_fix_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_scan_fwd_fix_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_seg_carry(const FwdParams&, hipStream_t) { return reached(); }
hipError_t dispatch_seg_summary_f32(const FwdParams&, int, bool, hipStream_t) { return reached(); }
hipError_t dispatch_seg_summary_bf16(const FwdParams&, int, bool, hipStream_t) { return reached(); }
hipError_t dispatch_seg_summary_reset_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_seg_summary_reset_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_fix_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_fix_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_fix_reset_f32(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_chunk_states_fix_reset_bf16(const FwdParams&, int, bool, hipStream_t) {
  return reached();
}
#define STUB_BWD(NAME)                                                                   \
  hipError_t NAME(const BwdParams&, int, bool, hipStream_t, hipEvent_t, hipEvent_t) { \
    return reached();                                                                    \
  }
STUB_BWD(dispatch_scan_bwd_f32_n16)
STUB_BWD(dispatch_scan_bwd_f32_n64)
STUB_BWD(dispatch_scan_bwd_bf16_n16)
STUB_BWD(dispatch_scan_bwd_bf16_n64)
STUB_BWD(dispatch_scan_bwd_reset_f32_n16)
STUB_BWD(dispatch_scan_bwd_reset_f32_n64)
STUB_BWD(dispatch_scan_bwd_reset_bf16_n16)
STUB_BWD(dispatch_scan_bwd_reset_bf16_n64)
#undef STUB_BWD
hipError_t dispatch_bwd_seg_summary(const BwdParams&, int, bool, hipStream_t) {
  return reached();
}
hipError_t dispatch_bwd_seg_carry(const BwdParams&, hipStream_t) { return reached(); }
hipError_t dispatch_state_update(const StepParams&, int, int, hipStream_t) { return reached(); }
hipError_t dispatch_state_update_complex(const CplxStepParams&, int, int, hipStream_t) {
  return reached();
}

}  // namespace mscan

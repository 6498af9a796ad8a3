// Carry between the segments of a segmented forward scan.
//
// Long sequences with few channels are split into segments that run in
// parallel.  A first launch of the forward kernel runs every segment from a
// zero state and gives each segment's end state and its delta sum.  This
// kernel walks the segments of each (channel, state) in order: the state
// entering segment s+1 is the one entering s, decayed by exp(A * sum of delta
// over s), plus s's end state from zero.  That is the associative combination
// of the (Abar, Bbar u) pairs the pages' parallel scan is built on
// (trishampatil essay, Part III §2), applied to whole segments; the chunking
// follows the same essay's Part III §4.  The state after the last segment is
// the sequence's last state.  A second launch of the forward kernel then
// corrects each segment's first chunks from its entering state.  A segment
// that contains a reset flag passes nothing on (its keep factor is 0).
#include "device_common.hpp"
#include "kernels.hpp"

namespace mscan {

// One thread per (channel, n).
static __global__ __launch_bounds__(256) void seg_carry_kernel(const FwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.nchannels * p.N) return;
  const int64_t c = i / p.N;
  const int n = (int)(i - c * p.N);
  const int64_t d = c % p.dim;
  const float a2 = p.A[d * p.N + n] * kLog2e;
  float H = p.h0 ? p.h0[c * p.N + n] : 0.0f;
  for (int64_t s = 0; s < p.nseg; ++s) {
    const int64_t k = c * p.nseg + s;
    p.seg_h0[k * p.N + n] = H;
    // a reset inside segment s cuts the carry (seg_keep = 0)
    const float decay = exp2f(a2 * p.seg_dsum[k]) * p.seg_keep[k];
    H = __builtin_fmaf(decay, H, p.seg_state[k * p.N + n]);
  }
  if (p.last_state) p.last_state[c * p.N + n] = H;
}

hipError_t dispatch_seg_carry(const FwdParams& p, hipStream_t s) {
  const int64_t total = p.nchannels * p.N;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(seg_carry_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mscan

// Issue-rate probes for the vector ALU of one GPU (used by `bench.py --probe`
// to measure the rates the scan kernels' ALU bound rests on; not part of the
// scan library).  Every thread runs 8 independent dependency chains of one
// instruction kind, so latency is hidden by the chains and by the many waves
// of the grid:
//   kind 0: v_fma_f32 / v_fmac_f32   x = x * 0.999 + 0.001
//   kind 1: v_exp_f32                x = exp2(-x)   (stays in [0.5, 1])
//   kind 2: v_mul_f32                x = x * 0.999
//   kind 3: v_rcp_f32                x = 1 / x
//   kind 4: v_fma_f32 with 1 chain per thread, kind 5 with 2 (dependency
//           latency: the issue rate when the next instruction needs the
//           previous one's result)
// Built with packed FP32 disabled, like the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int KIND, int CH = 8>
__global__ __launch_bounds__(256) void valu_probe_kernel(float* out, int iters) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.5f + 0.01f * (float)j + 1e-6f * (float)(gid & 255);
  for (int i = 0; i < iters * 8 / CH; ++i) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if constexpr (KIND == 0) x[j] = __builtin_fmaf(x[j], 0.999f, 0.001f);
      else if constexpr (KIND == 1) x[j] = __builtin_amdgcn_exp2f(-x[j]);
      else if constexpr (KIND == 2) x[j] = x[j] * 0.999f;
      else x[j] = __builtin_amdgcn_rcpf(x[j]);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[gid] = s;
}

}  // namespace

// Launches `blocks` blocks of 256 threads, each thread running `iters` x 8
// instructions of `kind` (in 8, 2 or 1 dependency chains), on `stream`, between the events `begin` and `end`
// (recorded on the same stream).  `out` holds blocks * 256 floats.  Returns 0
// on success, 1 for an unknown kind, 2 if a HIP call fails.
extern "C" int mscan_probe_valu(int kind, int blocks, int iters, float* out, void* stream,
                                void* begin, void* end) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipEventRecord(static_cast<hipEvent_t>(begin), s) != hipSuccess) return 2;
  switch (kind) {
    case 0: hipLaunchKernelGGL(valu_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 1: hipLaunchKernelGGL(valu_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 2: hipLaunchKernelGGL(valu_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 3: hipLaunchKernelGGL(valu_probe_kernel<3>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 4: hipLaunchKernelGGL((valu_probe_kernel<0, 1>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    case 5: hipLaunchKernelGGL((valu_probe_kernel<0, 2>), dim3(blocks), dim3(256), 0, s, out, iters); break;
    default: return 1;
  }
  if (hipGetLastError() != hipSuccess) return 2;
  if (hipEventRecord(static_cast<hipEvent_t>(end), s) != hipSuccess) return 2;
  return 0;
}

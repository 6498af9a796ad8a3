// One recurrent (decode) step of the selective SSM, in place on the state.
//
// The recurrent form h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = C_t h_t costs
// O(1) time and memory per step, which is what makes autoregressive
// inference cheap (paper-graph-ui summary of the Mamba paper, section 3.4,
// "What the recurrence computes"; chapterpal.com page, Knowl 1 step 4).
//
// Layout: state (batch, dim, N) with N contiguous.  G lanes (G = 16 or 64,
// G >= N) serve one channel, lane n owning h[n]: the state is read and
// written with coalesced accesses, and y = sum_n C[n] h[n] is a butterfly
// sum over the G lanes.  Lanes n >= N hold nothing and add zero.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mscan {

template <typename T, int G, bool ZOH>
__global__ __launch_bounds__(256) void state_update_kernel(const StepParams p) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n = (int)(gid % G);
  const int64_t c_raw = gid / G;
  const bool active = c_raw < p.nchannels;
  const int64_t c = active ? c_raw : p.nchannels - 1;
  const int64_t b = c / p.dim;
  const int64_t d = c - b * p.dim;
  const int N = p.N;
  const bool has_n = active && n < N;

  const float uv = Elem<T>::load1(static_cast<const T*>(p.u) + c);
  const float r = Elem<T>::load1(static_cast<const T*>(p.delta) + c) + (p.bias ? p.bias[d] : 0.0f);
  const float dt = p.softplus ? softplus(r) : r;

  float contrib = 0.0f;
  if (has_n) {
    const float An = p.A[d * N + n];
    const float Bn = Elem<T>::load1(static_cast<const T*>(p.B) + b * N + n);
    const float Cn = Elem<T>::load1(static_cast<const T*>(p.C) + b * N + n);
    const float z = dt * (An * kLog2e);
    const float a = fast_exp2(z);
    float coef;
    if constexpr (ZOH) coef = (__builtin_fabsf(An) < 1e-30f) ? dt : expm1_zoh(z, a) / An;
    else coef = dt;
    float* hp = p.state + c * N + n;
    const float h = __builtin_fmaf(a, *hp, coef * Bn * uv);
    *hp = h;
    contrib = Cn * h;
  }
  // sum over the G lanes of the channel (G divides 64, groups are aligned)
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) contrib += __shfl_xor(contrib, off);
  if (active && n == 0) {
    float y = __builtin_fmaf(p.D ? p.D[d] : 0.0f, uv, contrib);
    if (p.z) y *= silu(Elem<T>::load1(static_cast<const T*>(p.z) + c));
    Elem<T>::store1(static_cast<T*>(p.out) + c, y);
  }
}

template <typename T, int G>
static hipError_t launch_step(const StepParams& p, int disc, hipStream_t s) {
  const int64_t threads = p.nchannels * G;
  const int64_t blocks = (threads + 255) / 256;
  if (disc == 0)
    hipLaunchKernelGGL((state_update_kernel<T, G, true>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((state_update_kernel<T, G, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t dispatch_state_update(const StepParams& p, int dtype, int disc, hipStream_t stream) {
  if (dtype == 0)
    return p.N <= 16 ? launch_step<float, 16>(p, disc, stream) : launch_step<float, 64>(p, disc, stream);
  return p.N <= 16 ? launch_step<bf16_t, 16>(p, disc, stream) : launch_step<bf16_t, 64>(p, disc, stream);
}

}  // namespace mscan

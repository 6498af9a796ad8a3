// One recurrent (decode) step of the complex-valued selective SSM, in place
// on the complex state: autoregressive generation with the S4D-Lin-style
// complex A (paper-graph-ui summary, section 3.4, recurrent mode and "Real
// vs. Complex"; trishampatil essay, Part III).  Per channel (b, d) and state
// index n:
//   Abar = exp(delta A),  h <- Abar h + Ebar B u   (Ebar = (Abar - 1)/A, ZOH;
//   delta at A = 0, or delta for Euler),  y = Re(sum_n C[n] h[n]) + D u,
//   out = y * SiLU(z)
// -- the body of the complex forward's step loop applied to a stored state.
//
// Layout: state (batch, dim, N) interleaved (re, im) pairs with N
// contiguous; 16 lanes serve one channel, lane n owning h[n]; y is a
// butterfly sum over the 16 lanes.
#include "complex_common.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace mscan {

namespace {

constexpr int G = 16;

template <typename T, bool ZOH>
__global__ __launch_bounds__(256) void state_update_complex_kernel(const CplxStepParams p) {
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
    const float2 a = p.A[d * N + n];
    const float2 Bn = p.B[b * N + n];
    const float2 Cn = p.C[b * N + n];
    float2 em1;
    const float2 ab = cexp_expm1_scaled(dt, a.x * kLog2e, a.y * kInv2Pi, em1);
    const float2 Bu = cscale(Bn, uv);
    float2 bu;   // Ebar B u
    const bool tiny = __builtin_fabsf(a.x) < 1e-30f && __builtin_fabsf(a.y) < 1e-30f;
    if (ZOH && !tiny) {
      const float m2 = a.x * a.x + a.y * a.y;
      const float2 ia = make_float2(a.x / m2, -a.y / m2);
      bu = cmul(em1, cmul(ia, Bu));
    } else {
      bu = cscale(Bu, dt);
    }
    float2* hp = p.state + c * N + n;
    const float2 h = cfma(ab, *hp, bu);
    *hp = h;
    contrib = __builtin_fmaf(Cn.x, h.x, -Cn.y * h.y);   // Re(C h)
  }
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) contrib += __shfl_xor(contrib, off);
  if (active && n == 0) {
    float y = __builtin_fmaf(p.D ? p.D[d] : 0.0f, uv, contrib);
    if (p.z) y *= silu(Elem<T>::load1(static_cast<const T*>(p.z) + c));
    Elem<T>::store1(static_cast<T*>(p.out) + c, y);
  }
}

template <typename T>
hipError_t launch_step_complex(const CplxStepParams& p, int disc, hipStream_t s) {
  const int64_t blocks = (p.nchannels * G + 255) / 256;
  if (disc == 0)
    hipLaunchKernelGGL((state_update_complex_kernel<T, true>), dim3((unsigned)blocks), dim3(256),
                       0, s, p);
  else
    hipLaunchKernelGGL((state_update_complex_kernel<T, false>), dim3((unsigned)blocks), dim3(256),
                       0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t dispatch_state_update_complex(const CplxStepParams& p, int dtype, int disc,
                                         hipStream_t s) {
  return dtype == 0 ? launch_step_complex<float>(p, disc, s)
                    : launch_step_complex<bf16_t>(p, disc, s);
}

}  // namespace mscan

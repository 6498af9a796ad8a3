// Short causal depthwise convolution + SiLU: the stage that feeds the
// selective SSM in the Mamba block (chapterpal.com page, Knowl 3 "Mamba Block
// Architecture": a width-4 temporal convolution of the main branch, then
// SiLU, then the SSM; trishampatil essay, Part II §8, the same block).  Per
// channel (b, d) with W <= 4 taps:
//   pre_t = cb[d] + sum_k w[d, k] x_{t-(W-1)+k},   u_t = pre_t * sigmoid(pre_t)
// x before t = 0, and before the start of the current packed sequence when
// reset flags are given, counts as zero.  The backward recomputes pre from x
// instead of having it stored (the essay's Part III §4: cheap activations
// and the short convolution are recomputed, not saved).
//
// Layout: a block of 256 threads covers 2048 consecutive steps of one
// channel, 8 per thread: the thread's own 8 x values come in one vector
// load, the 3 before (and, in the backward, the 3 after) from the
// neighbouring threads' runs through the cache.  Both kernels are bound by
// HBM traffic: the forward reads x and writes u once; the backward reads x
// and du and writes dx once, and sums dw / dcb over the block before one
// atomic per tap.
#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_fwd_impl.hpp"

namespace mscan {

namespace {

constexpr int kRun = kConvRun;             // steps per thread
constexpr int kTile = kConvTile;           // steps per block
constexpr int kTaps = 4;                   // taps held per thread (W <= 4)

// Taps right-aligned to x_{t-3..t}: tap j multiplies x_{t-3+j}.
__device__ __forceinline__ void load_taps(const ConvParams& p, int64_t d, float (&w4)[kTaps]) {
#pragma unroll
  for (int j = 0; j < kTaps; ++j) {
    const int k = j - (kTaps - p.W);
    w4[j] = k >= 0 ? p.w[d * p.W + k] : 0.0f;
  }
}

// Start of the packed sequence that step t0 - 3 + i belongs to, for the
// steps of a window [t0 - 3, t0 - 3 + NW): the last flagged step <= it
// (INT64_MIN when none is flagged in the window).
template <int NW>
__device__ __forceinline__ void seq_starts(const uint8_t* __restrict__ rrow, int64_t t0, int64_t L,
                                           int64_t (&st)[NW]) {
  int64_t last = INT64_MIN;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int64_t q = t0 - 3 + i;
    if (q >= 0 && q < L && rrow[q] != 0) last = q;
    st[i] = last;
  }
}

template <typename T, bool VEC, bool RST>
__global__ __launch_bounds__(256) void conv1d_silu_fwd_kernel(const ConvParams p) {
  const int64_t c = blockIdx.x / p.tiles;
  const int64_t t0 = (blockIdx.x - c * p.tiles) * (int64_t)kTile + threadIdx.x * kRun;
  if (t0 >= p.L) return;
  const int64_t b = c / p.dim, d = c - b * p.dim;
  const int64_t L = p.L;
  const T* __restrict__ xr = static_cast<const T*>(p.x) + c * L;
  float w4[kTaps];
  load_taps(p, d, w4);
  const float cb = p.b ? p.b[d] : 0.0f;

  float xv[3 + kRun];   // x_{t0-3} .. x_{t0+7}
#pragma unroll
  for (int i = 0; i < 3; ++i) xv[i] = t0 - 3 + i >= 0 ? Elem<T>::load1(xr + t0 - 3 + i) : 0.0f;
  const bool full = VEC && t0 + kRun <= L;
  {
    float m[kRun];
    load_items<T, kRun>(xr, t0, L, full, m);
#pragma unroll
    for (int i = 0; i < kRun; ++i) xv[3 + i] = m[i];
  }
  int64_t st[3 + kRun];
  if constexpr (RST) seq_starts<3 + kRun>(p.reset + b * L, t0, L, st);

  float u[kRun];
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    float pre = cb;
#pragma unroll
    for (int j = 0; j < kTaps; ++j) {
      // x_{t0+i-3+j} is window slot i+j; it counts if it is in the sequence of t0+i
      const bool ok = !RST || t0 + i - 3 + j >= st[3 + i];
      pre = ok ? __builtin_fmaf(w4[j], xv[i + j], pre) : pre;
    }
    u[i] = silu(pre);
  }
  store_items<T, kRun>(static_cast<T*>(p.u) + c * L, t0, L, full, u);
}

template <typename T, bool VEC, bool RST>
__global__ __launch_bounds__(256) void conv1d_silu_bwd_kernel(const ConvParams p) {
  __shared__ float red[4][kTaps + 1];
  const int64_t c = blockIdx.x / p.tiles;
  const int64_t t0 = (blockIdx.x - c * p.tiles) * (int64_t)kTile + threadIdx.x * kRun;
  const int64_t b = c / p.dim, d = c - b * p.dim;
  const int64_t L = p.L;
  float w4[kTaps];
  load_taps(p, d, w4);
  const float cb = p.b ? p.b[d] : 0.0f;
  float dwp[kTaps] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dbp = 0.0f;

  if (t0 < L) {
    const T* __restrict__ xr = static_cast<const T*>(p.x) + c * L;
    const float* __restrict__ gr = p.du + c * L;
    const bool full = VEC && t0 + kRun <= L;
    // x_{t0-3} .. x_{t0+10} and du_{t0} .. du_{t0+10}
    float xv[3 + kRun + 3], g[kRun + 3];
#pragma unroll
    for (int i = 0; i < 3; ++i) xv[i] = t0 - 3 + i >= 0 ? Elem<T>::load1(xr + t0 - 3 + i) : 0.0f;
    {
      float m[kRun], gm[kRun];
      load_items<T, kRun>(xr, t0, L, full, m);
      load_items<float, kRun>(gr, t0, L, full, gm);
#pragma unroll
      for (int i = 0; i < kRun; ++i) {
        xv[3 + i] = m[i];
        g[i] = gm[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int64_t t = t0 + kRun + i;
      xv[3 + kRun + i] = t < L ? Elem<T>::load1(xr + t) : 0.0f;
      g[kRun + i] = t < L ? gr[t] : 0.0f;
    }
    int64_t st[3 + kRun + 3];
    if constexpr (RST) seq_starts<3 + kRun + 3>(p.reset + b * L, t0, L, st);

    // dpre at steps t0 .. t0+10 (zero past L: du is zero there)
    float dpre[kRun + 3];
#pragma unroll
    for (int i = 0; i < kRun + 3; ++i) {
      float pre = cb;
#pragma unroll
      for (int j = 0; j < kTaps; ++j) {
        const bool ok = !RST || t0 + i - 3 + j >= st[3 + i];
        pre = ok ? __builtin_fmaf(w4[j], xv[i + j], pre) : pre;
      }
      const float sg = sigmoid(pre);
      dpre[i] = g[i] * sg * __builtin_fmaf(pre, 1.0f - sg, 1.0f);
    }
    // dx_s = sum_j w4[j] dpre_{s+3-j} over the taps that reach step s
    float dx[kRun];
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < kTaps; ++j) {
        const int o = i + 3 - j;                  // output step t0 + o
        const bool ok = !RST || t0 + i >= st[3 + o];
        acc = ok ? __builtin_fmaf(w4[j], dpre[o], acc) : acc;
      }
      dx[i] = acc;
    }
    store_items<float, kRun>(p.dx + c * L, t0, L, full, dx);
    // the thread's share of dw, dcb: outputs t0 .. t0+7
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      dbp += dpre[i];
#pragma unroll
      for (int j = 0; j < kTaps; ++j) {
        const bool ok = !RST || t0 + i - 3 + j >= st[3 + i];
        dwp[j] = ok ? __builtin_fmaf(dpre[i], xv[i + j], dwp[j]) : dwp[j];
      }
    }
  }
  // sum over the block: within each wave, then over the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
    for (int j = 0; j < kTaps; ++j) dwp[j] += __shfl_xor(dwp[j], off);
    dbp += __shfl_xor(dbp, off);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int j = 0; j < kTaps; ++j) red[wave][j] = dwp[j];
    red[wave][kTaps] = dbp;
  }
  __syncthreads();
  if (threadIdx.x < kTaps + 1) {
    const int j = threadIdx.x;
    const float v = red[0][j] + red[1][j] + red[2][j] + red[3][j];
    if (j < kTaps) {
      const int k = j - (kTaps - p.W);
      if (k >= 0) unsafeAtomicAdd(p.dw + d * p.W + k, v);
    } else if (p.db) {
      unsafeAtomicAdd(p.db + d, v);
    }
  }
}

// dw, dcb are accumulated: cleared first by a plain kernel (no memset node).
__global__ __launch_bounds__(256) void conv_zero_kernel(const ConvParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < p.dim * p.W) p.dw[i] = 0.0f;
  if (p.db && i < p.dim) p.db[i] = 0.0f;
}

template <typename T>
hipError_t conv_fwd_t(const ConvParams& p, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)(p.nchannels * p.tiles)), block(256);
  if (p.reset) {
    if (vec) hipLaunchKernelGGL((conv1d_silu_fwd_kernel<T, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((conv1d_silu_fwd_kernel<T, false, true>), grid, block, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((conv1d_silu_fwd_kernel<T, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((conv1d_silu_fwd_kernel<T, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t conv_bwd_t(const ConvParams& p, bool vec, hipStream_t s) {
  const int64_t nz = p.dim * p.W;
  hipLaunchKernelGGL(conv_zero_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(p.nchannels * p.tiles)), block(256);
  if (p.reset) {
    if (vec) hipLaunchKernelGGL((conv1d_silu_bwd_kernel<T, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((conv1d_silu_bwd_kernel<T, false, true>), grid, block, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((conv1d_silu_bwd_kernel<T, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((conv1d_silu_bwd_kernel<T, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t dispatch_conv_fwd(const ConvParams& p, int dtype, bool vec, hipStream_t s) {
  return dtype == 0 ? conv_fwd_t<float>(p, vec, s) : conv_fwd_t<bf16_t>(p, vec, s);
}

hipError_t dispatch_conv_bwd(const ConvParams& p, int dtype, bool vec, hipStream_t s) {
  return dtype == 0 ? conv_bwd_t<float>(p, vec, s) : conv_bwd_t<bf16_t>(p, vec, s);
}

}  // namespace mscan

// Selective-scan backward for gfx950: recompute the states, run the adjoint
// recurrence in reverse time, and form every input gradient.
//
// The pages only say that the backward recomputes the (B, L, D, N) states
// from the inputs instead of saving them (paper-graph-ui summary of the Mamba
// paper, section 3.4, "Recomputation for the backward pass"; chapterpal.com
// page, Knowl 2 item 2).  The gradient formulas are the chain rule of the
// forward (see scan_fwd.hip); with gy_t = dout_t * SiLU(z_t):
//   gh_t[n] = C_t[n] gy_t + Abar_{t+1}[n] gh_{t+1}[n]      (reverse recurrence)
//   du_t    = D gy_t + sum_n gh_t Bbar_t
//   ddelta  = softplus'(r_t) * sum_n gh_t (h_{t-1} A Abar_t + u_t dBbar/ddelta)
//   dA[d,n] = sum_{b,t} gh_t (h_{t-1} delta_t Abar_t + u_t dBbar/dA)
//   dB_t[n] = sum_d gh_t u_t Bbar_t/B_t,  dC_t[n] = sum_d gy_t h_t[n]
//   dz_t    = dout_t y_t SiLU'(z_t),  dD = sum gy u,  ddelta_bias = sum ddelta
// With g_t = Abar_t gh_t the reverse recurrence is g_t = Abar_t (g_{t+1} + e_t),
// e_t = C_t gy_t: an affine map per step, so it scans like the forward.
//
// Three launches:
//   1. chunk_states (scan_fwd.hip, states-only mode): the forward state at the
//      start of every chunk of R*K steps, into the workspace;
//   2. this kernel: chunks in reverse order; per chunk and state index n,
//      replay the forward from the stored chunk-start state (pass 1, DPP scan,
//      pass 2 keeping h in registers), then the reverse adjoint (reverse pass
//      1, DPP suffix scan with the carry from the later chunk, reverse pass 2)
//      and the gradient terms.  dB/dC are summed over the block's channels in
//      LDS and written as one partial per channel group; dA, dD, ddelta_bias
//      are summed over the channel's lanes and written per batch row.  No
//      global atomics: the result is deterministic;
//   3. bwd_reduce: sums the partials.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mscan {

// Lane i receives lane i+1 of its group; lane R-1 of the group receives `last`.
template <int R>
__device__ __forceinline__ float group_shift_left(float v, float last) {
  if constexpr (R == 16) {
    return dpp_mov<0x101 /*row_shl:1*/>(last, v);
  } else {
    float s = dpp_mov<0x130 /*wave_shl:1*/>(last, v);
    if constexpr (R == 32) s = ((__lane_id() & 31) == 31) ? last : s;
    return s;
  }
}

template <int CTRL>
__device__ __forceinline__ void affine_step_rev(float& A, float& B) {
  float Ap = dpp_mov<CTRL>(1.0f, A);
  float Bp = dpp_mov<CTRL>(0.0f, B);
  B = __builtin_fmaf(A, Bp, B);
  A = A * Ap;
}

// Inclusive suffix scan of affine pairs over groups of R lanes: lane i ends
// with the composition of lanes i..R-1, later lanes applied first.  Within a
// 16-lane row DPP row_shl; across rows a cross-lane read of the next row's
// first lane (which then holds that row's total).
template <int R>
__device__ __forceinline__ void affine_suffix_scan(float& A, float& B) {
  affine_step_rev<0x101>(A, B);   // row_shl:1
  affine_step_rev<0x102>(A, B);   // row_shl:2
  affine_step_rev<0x104>(A, B);   // row_shl:4
  affine_step_rev<0x108>(A, B);   // row_shl:8
  if constexpr (R >= 32) {
    const int lane = __lane_id();
    const bool take = ((lane >> 4) & 1) == 0;         // lower row of each 32-lane pair
    const int src = (lane & ~15) + 16;
    float Ap = __shfl(A, src & 63);
    float Bp = __shfl(B, src & 63);
    if (take) {
      B = __builtin_fmaf(A, Bp, B);
      A = A * Ap;
    }
  }
  if constexpr (R == 64) {
    const int lane = __lane_id();
    float Ap = __shfl(A, 32);
    float Bp = __shfl(B, 32);
    if (lane < 32) {
      B = __builtin_fmaf(A, Bp, B);
      A = A * Ap;
    }
  }
}

template <typename T, int R, int K, int NT, bool ZOH, bool VEC>
__global__ __launch_bounds__(kBlock) void scan_bwd_kernel(const BwdParams p) {
  constexpr int CPW = 64 / R;
  constexpr int CPB = (kBlock / 64) * CPW;
  constexpr int TCH = R * K;   // steps per chunk
  __shared__ float acc[2][2][TCH];   // [buffer][dB, dC][step in chunk]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % R;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = blk / p.groups;
  const int64_t grp = blk - b * p.groups;
  const int64_t d_raw = grp * CPB + wave * CPW + lane / R;
  const bool active = d_raw < p.dim;
  const int64_t d = active ? d_raw : p.dim - 1;
  const int64_t c = b * p.dim + d;
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t nchunks = p.nchunks;

  const T* __restrict__ u_row = static_cast<const T*>(p.u) + c * L;
  const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + c * L;
  const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + c * L : nullptr;
  const T* __restrict__ do_row = static_cast<const T*>(p.dout) + c * L;
  const T* __restrict__ B_b = static_cast<const T*>(p.B) + b * N * L;
  const T* __restrict__ C_b = static_cast<const T*>(p.C) + b * N * L;
  const float* __restrict__ A_d = p.A + d * N;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  float* __restrict__ part_bc = p.part_bc + (b * p.groups + grp) * 2 * N * L;

  for (int i = threadIdx.x; i < 2 * 2 * TCH; i += kBlock) (&acc[0][0][0])[i] = 0.0f;
  __syncthreads();

  float gcarry[NT];   // adjoint carried in from the later chunk: Abar gh at its first step
  float dA1[NT];      // this lane's share of dA[d, n]
#pragma unroll
  for (int n = 0; n < NT; ++n) gcarry[n] = dA1[n] = 0.0f;
  float dD_acc = 0.0f, db_acc = 0.0f;
  int buf = 0;

  for (int64_t ch = nchunks - 1; ch >= 0; --ch) {
    const int64_t tl = ch * TCH + (int64_t)j * K;
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    const float* __restrict__ hs_chunk = p.chunk_states + (c * nchunks + ch) * N;

    float uv[K], dt[K], gy[K], yv[K], du[K], gdt[K];
    {
      float raw[K], dov[K];
      load_run<T, K, VEC>(u_row, tl, L, uv);
      load_run<T, K, VEC>(dl_row, tl, L, raw);
      load_run<T, K, VEC>(do_row, tl, L, dov);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float r = raw[k] + bias;
        float s = p.softplus ? softplus(r) : r;
        dt[k] = (k < nvalid) ? s : 0.0f;
        gy[k] = dov[k];
      }
      if (z_row) {
        float zv[K];
        load_run<T, K, VEC>(z_row, tl, L, zv);
#pragma unroll
        for (int k = 0; k < K; ++k) gy[k] *= silu(zv[k]);
      }
    }
    float dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      dsum += dt[k];
      yv[k] = Dd * uv[k];
      du[k] = Dd * gy[k];
      gdt[k] = 0.0f;
      dD_acc = __builtin_fmaf(gy[k], uv[k], dD_acc);
    }

#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n < N) {
        const float An = A_d[n];
        const float a2 = An * kLog2e;
        const bool tiny = ZOH && __builtin_fabsf(An) < 1e-30f;
        const float ia = tiny ? 0.0f : fast_rcp(An);
        float Bv[K], Cv[K];
        load_run<T, K, VEC>(B_b + (int64_t)n * L, tl, L, Bv);
        load_run<T, K, VEC>(C_b + (int64_t)n * L, tl, L, Cv);

        // ---- forward replay of this chunk for state index n ----
        float a[K], beta[K], hv[K];
        float agg = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          a[k] = fast_exp2(dt[k] * a2);
          float coef;
          if constexpr (ZOH) coef = tiny ? dt[k] : (a[k] - 1.0f) * ia;
          else coef = dt[k];
          beta[k] = coef * Bv[k] * uv[k];
          agg = __builtin_fmaf(a[k], agg, beta[k]);
        }
        const float Alane = fast_exp2(a2 * dsum);
        float Ag = Alane;
        affine_scan_inclusive<R>(Ag, agg);
        const float h_in = hs_chunk[n];
        const float hend = __builtin_fmaf(Ag, h_in, agg);
        const float hstart = group_shift_right<R>(hend, h_in);
        {
          float h = hstart;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            h = __builtin_fmaf(a[k], h, beta[k]);
            hv[k] = h;
            yv[k] = __builtin_fmaf(Cv[k], h, yv[k]);
          }
        }

        // ---- reverse adjoint: g_t = Abar_t (g_{t+1} + C_t gy_t) ----
        float gagg = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) gagg = a[k] * (__builtin_fmaf(Cv[k], gy[k], gagg));
        float As = Alane;
        affine_suffix_scan<R>(As, gagg);
        const float gstart = __builtin_fmaf(As, gcarry[n], gagg);   // g leaving this lane leftwards
        float g = group_shift_left<R>(gstart, gcarry[n]);           // g entering from the right
        gcarry[n] = group_first<R>(gstart);
        float dA2 = 0.0f;   // sum of gh * Bbar * u, scaled by -1/A below (ZOH)

#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
          const float gh = __builtin_fmaf(Cv[k], gy[k], g);          // dL/dh_t
          const float hprev = (k == 0) ? hstart : hv[k - 1];
          const float P = gh * a[k];
          float coef, dbdd;
          if constexpr (ZOH) {
            coef = tiny ? dt[k] : (a[k] - 1.0f) * ia;
            dbdd = a[k] * Bv[k];                                     // dBbar/ddelta
          } else {
            coef = dt[k];
            dbdd = Bv[k];
          }
          // ddelta: gh * (hprev * A * Abar + u * dBbar/ddelta)
          gdt[k] = __builtin_fmaf(P * hprev, An, gdt[k]);
          gdt[k] = __builtin_fmaf(gh * uv[k], dbdd, gdt[k]);
          // dA: gh * hprev * delta * Abar + gh * u * dBbar/dA,
          // ZOH dBbar/dA = (delta*Abar*B - Bbar)/A  (limit delta^2 B / 2 at A = 0)
          dA1[n] = __builtin_fmaf(dt[k], P * hprev, dA1[n]);
          if constexpr (ZOH) {
            const float gu = gh * uv[k];
            if (tiny) {
              dA1[n] = __builtin_fmaf(gu, 0.5f * dt[k] * dt[k] * Bv[k], dA1[n]);
            } else {
              dA1[n] = __builtin_fmaf(gu * dt[k], a[k] * Bv[k] * ia, dA1[n]);
              dA2 = __builtin_fmaf(gh, beta[k], dA2);
            }
          }
          const float s = gh * coef;
          du[k] = __builtin_fmaf(s, Bv[k], du[k]);
          if (active) {
            atomicAdd(&acc[buf][0][j * K + k], s * uv[k]);
            atomicAdd(&acc[buf][1][j * K + k], gy[k] * hv[k]);
          }
          g = P;
        }
        if constexpr (ZOH) dA1[n] = __builtin_fmaf(-dA2, ia, dA1[n]);

        // ---- publish this block's dB/dC partial for (n, chunk) ----
        __syncthreads();
        for (int i = threadIdx.x; i < 2 * TCH; i += kBlock) {
          const int which = i / TCH, tt = i - which * TCH;
          const int64_t t = ch * TCH + tt;
          float v = acc[buf][which][tt];
          acc[buf][which][tt] = 0.0f;
          if (t < L) part_bc[((int64_t)which * N + n) * L + t] = v;
        }
        buf ^= 1;
      }
    }

    // ---- per-step outputs ----
    float sig[K];
    {
      float raw[K];
      load_run<T, K, VEC>(dl_row, tl, L, raw);
#pragma unroll
      for (int k = 0; k < K; ++k) sig[k] = p.softplus ? sigmoid(raw[k] + bias) : 1.0f;
    }
    float ddl[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      ddl[k] = (k < nvalid) ? gdt[k] * sig[k] : 0.0f;
      db_acc += ddl[k];
    }
    if (active) {
      float* du_row = p.du + c * L;
      float* dd_row = p.ddelta + c * L;
      store_run<float, K, VEC>(du_row, tl, L, du);
      store_run<float, K, VEC>(dd_row, tl, L, ddl);
    }
    if (z_row) {
      float zv[K], dov[K];
      load_run<T, K, VEC>(z_row, tl, L, zv);
      load_run<T, K, VEC>(do_row, tl, L, dov);
      float dzv[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float sg = sigmoid(zv[k]);
        dzv[k] = dov[k] * yv[k] * sg * __builtin_fmaf(zv[k], 1.0f - sg, 1.0f);
      }
      if (active) store_run<float, K, VEC>(p.dz + c * L, tl, L, dzv);
    }
  }

  // ---- per-channel reductions over the channel's lanes ----
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (n < N) {
      const float s = group_sum<R>(dA1[n]);
      if (active && j == 0) p.part_a[c * N + n] = s;
      if (active && j == 0 && p.dh0) p.dh0[c * N + n] = gcarry[n];
    }
  }
  const float sD = group_sum<R>(dD_acc);
  const float sb = group_sum<R>(db_acc);
  if (active && j == 0) {
    p.part_d[c * 2 + 0] = sD;
    p.part_d[c * 2 + 1] = sb;
  }
}

// Sums the partials: dB/dC over channel groups, dA/dD/ddelta_bias over batch.
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const BwdParams p) {
  const int64_t total = p.batch * 2 * p.N * p.L;   // (batch, 2, N, L)
  const int64_t NL = (int64_t)p.N * p.L;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / (2 * NL);
    const int64_t rest = i - b * 2 * NL;           // which * NL + n * L + t
    const float* src = p.part_bc + b * p.groups * 2 * NL + rest;
    float s = 0.0f;
    for (int64_t g = 0; g < p.groups; ++g) s += src[g * 2 * NL];
    const int64_t which = rest / NL;
    float* dst = (which == 0 ? p.dB : p.dC) + b * NL + (rest - which * NL);
    *dst = s;
  }
}

__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(const BwdParams p) {
  const int64_t nA = p.dim * p.N;
  const int64_t total = nA + 2 * p.dim;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    if (i < nA) {
      for (int64_t b = 0; b < p.batch; ++b) s += p.part_a[b * nA + i];
      p.dA[i] = s;
    } else {
      const int64_t k = i - nA;          // d * 2 + which
      const int64_t d = k >> 1, which = k & 1;
      for (int64_t b = 0; b < p.batch; ++b) s += p.part_d[(b * p.dim + d) * 2 + which];
      float* dst = which == 0 ? p.dD : p.dbias;
      if (dst) dst[d] = s;
    }
  }
}

hipError_t launch_bwd_reduce(const BwdParams& p, hipStream_t s) {
  const int64_t total = p.batch * 2 * p.N * p.L;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tp = p.dim * p.N + 2 * p.dim;
  int64_t pb = (tp + 255) / 256;
  if (pb > 65536) pb = 65536;
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)pb), dim3(256), 0, s, p);
  return hipGetLastError();
}

int64_t bwd_groups(int64_t dim, int lanes) {
  const int64_t cpb = (kBlock / 64) * (64 / lanes);
  return (dim + cpb - 1) / cpb;
}

template <typename T, int R, int NT, bool ZOH, bool VEC>
static hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t nblocks = p.batch * p.groups;
  hipLaunchKernelGGL((scan_bwd_kernel<T, R, kItemsBwd, NT, ZOH, VEC>), dim3((unsigned)nblocks),
                     dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

template <typename T, int R, int NT, bool ZOH>
static hipError_t bwd_v(const BwdParams& p, bool vec, hipStream_t s) {
  return vec ? launch_bwd<T, R, NT, ZOH, true>(p, s) : launch_bwd<T, R, NT, ZOH, false>(p, s);
}

template <typename T, int R, int NT>
static hipError_t bwd_d(const BwdParams& p, int disc, bool vec, hipStream_t s) {
  return disc == 0 ? bwd_v<T, R, NT, true>(p, vec, s) : bwd_v<T, R, NT, false>(p, vec, s);
}

template <typename T, int R>
static hipError_t bwd_n(const BwdParams& p, int disc, bool vec, hipStream_t s) {
  return p.N <= 16 ? bwd_d<T, R, 16>(p, disc, vec, s) : bwd_d<T, R, 64>(p, disc, vec, s);
}

template <typename T>
static hipError_t bwd_r(const BwdParams& p, int disc, int lanes, bool vec, hipStream_t s) {
  switch (lanes) {
    case 16: return bwd_n<T, 16>(p, disc, vec, s);
    case 32: return bwd_n<T, 32>(p, disc, vec, s);
    default: return bwd_n<T, 64>(p, disc, vec, s);
  }
}

hipError_t dispatch_scan_bwd(const BwdParams& p, int dtype, int disc, int lanes, bool vec,
                             hipStream_t stream) {
  return dtype == 0 ? bwd_r<float>(p, disc, lanes, vec, stream)
                    : bwd_r<bf16_t>(p, disc, lanes, vec, stream);
}

}  // namespace mscan

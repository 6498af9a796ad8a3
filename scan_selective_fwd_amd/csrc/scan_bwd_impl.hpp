// Selective-scan backward for gfx950 (kernel template; instantiated per
// element type in scan_bwd_{f32,bf16}.hip): recompute the states, run the
// adjoint recurrence in reverse time, and form every input gradient.
//
// The pages only say that the backward recomputes the (B, L, D, N) states
// from the inputs instead of saving them (paper-graph-ui summary of the Mamba
// paper, section 3.4, "Recomputation for the backward pass"; chapterpal.com
// page, Knowl 2 item 2).  The gradient formulas are the chain rule of the
// forward (scan_fwd_impl.hpp); with gy_t = dout_t * SiLU(z_t):
//   gh_t[n] = C_t[n] gy_t + Abar_{t+1}[n] gh_{t+1}[n]      (reverse recurrence)
//   du_t    = D gy_t + sum_n gh_t Bbar_t
//   ddelta  = softplus'(r_t) * sum_n gh_t (h_{t-1} A Abar_t + u_t dBbar/ddelta)
//   dA[d,n] = sum_{b,t} gh_t (h_{t-1} delta_t Abar_t + u_t dBbar/dA)
//   dB_t[n] = sum_d gh_t u_t Bbar_t/B_t,  dC_t[n] = sum_d gy_t h_t[n]
//   dz_t    = dout_t y_t SiLU'(z_t),  dD = sum gy u,  ddelta_bias = sum ddelta
// With g_t = Abar_t gh_t the reverse recurrence is g_t = Abar_t (g_{t+1} + e_t),
// e_t = C_t gy_t: an affine map per step, so it scans like the forward, with
// suffix instead of prefix composition.
//
// Launches (api.cpp): a zero fill of the accumulated gradients; the forward
// kernel in states-only mode (the state at every chunk start, into the
// workspace); then this kernel.  Here a block serves 16 channels of one batch
// row (4 per wave, 16 lanes each, 8 steps per lane: 128-step chunks) and walks
// the chunks from last to first.  Per chunk and state index n it replays the
// forward from the stored chunk-start state (pass 1, DPP prefix scan, pass 2
// keeping h in registers), then the adjoint (reverse pass 1, DPP suffix scan
// with the carry from the later chunk, reverse pass 2) and the gradient
// terms.  The B/C chunk and the chunk-start states are staged in LDS once per
// block.  dB/dC are summed over the wave's 4 channels with gfx950 permlane
// swaps, over the block's waves with LDS float adds, and once per chunk into
// global memory with float atomics.  dA, dD, ddelta_bias are summed over the
// channel's lanes and atomically over batch rows.  Atomics make the result
// deterministic only up to float32 rounding order.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_fwd_impl.hpp"
#include "tile_stage.hpp"

namespace mscan {

// Lane i receives lane i+1 of its 16-lane row; lane 15 receives `last`.
__device__ __forceinline__ float row_shift_left(float v, float last) {
  return dpp_mov<0x101 /*row_shl:1*/>(last, v);
}

template <typename T, int NT, bool ZOH, bool VEC>
__global__ __launch_bounds__(kBlock) void scan_bwd_kernel(const BwdParams p) {
  constexpr int R = 16;
  constexpr int K = kItemsBwd;
  static_assert(K == 8, "the row reduce-scatter assumes 8 steps per lane");
  constexpr int CPW = 64 / R;
  constexpr int CPB = (kBlock / 64) * CPW;
  constexpr int TCH = R * K;
  constexpr bool TILE = (NT == 16);
  __shared__ float4 tile_mem[2][TILE ? 2 * NT * TCH / 4 : 1];
  __shared__ float hst[2][CPB][NT];          // chunk-start states
  __shared__ float acc[2][NT][TCH];          // dB, dC summed over the block's channels
  __shared__ float a2s[CPB][NT], ias[CPB][NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane % R;
  const int row = lane / R;
  const int cl = wave * CPW + row;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = blk / p.groups;
  const int64_t grp = blk - b * p.groups;
  const int64_t d_raw = grp * CPB + cl;
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
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;

  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    const float a = (dd < p.dim && n < N) ? p.A[dd * N + n] : -1.0f;
    a2s[ci][n] = a * kLog2e;
    ias[ci][n] = __builtin_fabsf(a) < 1e-30f ? 0.0f : 1.0f / a;
  }
  for (int i = tid; i < 2 * NT * TCH; i += kBlock) (&acc[0][0][0])[i] = 0.0f;

  // chunk-start states of this block's channels for chunk `ch`
  auto load_states = [&](int64_t ch, float (&dst)[(CPB * NT + kBlock - 1) / kBlock]) {
#pragma unroll
    for (int r = 0; r < (CPB * NT + kBlock - 1) / kBlock; ++r) {
      const int i = r * kBlock + tid;
      const int ci = i / NT, n = i - ci * NT;
      const int64_t dd = grp * CPB + ci;
      dst[r] = (i < CPB * NT && dd < p.dim && n < N)
                   ? p.chunk_states[((b * p.dim + dd) * nchunks + ch) * N + n] : 0.0f;
    }
  };
  auto store_states = [&](int bufi, const float (&src)[(CPB * NT + kBlock - 1) / kBlock]) {
#pragma unroll
    for (int r = 0; r < (CPB * NT + kBlock - 1) / kBlock; ++r) {
      const int i = r * kBlock + tid;
      if (i < CPB * NT) (&hst[bufi][0][0])[i] = src[r];
    }
  };

  TileStager<T, TCH, K, NT, TILE ? 2 * NT : 1, kBlock> stage;
  float hreg[(CPB * NT + kBlock - 1) / kBlock];
  {
    const int64_t last = nchunks - 1;
    const bool full_last = VEC && last * TCH + TCH <= L;
    if constexpr (TILE) {
      stage.load(B_b, C_b, N, L, last * TCH, full_last, tid);
      stage.store(reinterpret_cast<float*>(tile_mem[0]), N, tid);
    }
    load_states(last, hreg);
    store_states(0, hreg);
  }
  __syncthreads();

  float gcarry[NT];   // adjoint entering each chunk from the later one
  float dA1[NT];      // this lane's share of dA[d, n]
#pragma unroll
  for (int n = 0; n < NT; ++n) gcarry[n] = dA1[n] = 0.0f;
  float dD_acc = 0.0f, db_acc = 0.0f;

  for (int64_t ch = nchunks - 1; ch >= 0; --ch) {
    const int buf = (int)((nchunks - 1 - ch) & 1);
    const int64_t t0 = ch * TCH;
    const int64_t tl = t0 + (int64_t)j * K;
    const bool full = VEC && t0 + TCH <= L;
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    if (ch > 0) {
      if constexpr (TILE) stage.load(B_b, C_b, N, L, t0 - TCH, VEC, tid);   // earlier chunks are full
      load_states(ch - 1, hreg);
    }

    float uv[K], dt[K], gy[K], yv[K], du[K], gdt[K], sig[K];
    {
      float raw[K], dov[K];
      load_items<T, K>(u_row, tl, L, full, uv);
      load_items<T, K>(dl_row, tl, L, full, raw);
      load_items<T, K>(do_row, tl, L, full, dov);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float r = raw[k] + bias;
        const float s = p.softplus ? softplus(r) : r;
        sig[k] = p.softplus ? sigmoid(r) : 1.0f;
        dt[k] = (k < nvalid) ? s : 0.0f;
        gy[k] = dov[k];
      }
      if (z_row) {
        float zv[K];
        load_items<T, K>(z_row, tl, L, full, zv);
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

    const float* tB = reinterpret_cast<const float*>(tile_mem[buf]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n < N) {
        const float An = p.A[d * N + n];
        const float a2 = a2s[cl][n];
        const float ia = ias[cl][n];
        const bool tiny = ZOH && ia == 0.0f;
        const bool any_tiny = __builtin_amdgcn_ballot_w64(tiny) != 0;
        float Bv[K], Cv[K];
        if constexpr (TILE) {
          tile_read<K>(tB + n * TCH, j, Bv);
          tile_read<K>(tB + (NT + n) * TCH, j, Cv);
        } else {
          load_items<T, K>(B_b + (int64_t)n * L, tl, L, full, Bv);
          load_items<T, K>(C_b + (int64_t)n * L, tl, L, full, Cv);
        }

        // ---- forward replay of this chunk for state index n ----
        float a[K], beta[K], hv[K];
        float agg = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          a[k] = fast_exp2(dt[k] * a2);
          if constexpr (ZOH) {
            if (!any_tiny) {
              const float q = Bv[k] * (uv[k] * ia);
              beta[k] = __builtin_fmaf(a[k], q, -q);
            } else {
              const float coef = tiny ? dt[k] : (a[k] - 1.0f) * ia;
              beta[k] = coef * Bv[k] * uv[k];
            }
          } else {
            beta[k] = dt[k] * Bv[k] * uv[k];
          }
          agg = __builtin_fmaf(a[k], agg, beta[k]);
        }
        const float Alane = fast_exp2(a2 * dsum);
        float Ag = Alane;
        affine_scan_inclusive_fused<R>(Ag, agg);
        const float h_in = hst[buf][cl][n];
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
        float e[K];
        float gagg = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
          e[k] = Cv[k] * gy[k];
          gagg = a[k] * (e[k] + gagg);
        }
        float As = Alane;
        affine_suffix_scan_row_fused(As, gagg);
        const float gstart = __builtin_fmaf(As, gcarry[n], gagg);   // leaving this lane leftwards
        float g = row_shift_left(gstart, gcarry[n]);                 // entering from the right
        gcarry[n] = group_first<R>(gstart);

        float dBv[K], dCv[K];
        float dA2 = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
          const float gh = e[k] + g;                      // dL/dh_t
          const float hprev = (k == 0) ? hstart : hv[k - 1];
          const float P = gh * a[k];
          const float gu = gh * uv[k];
          float coef, dbdd;
          if constexpr (ZOH) {
            coef = __builtin_fmaf(a[k], ia, -ia);                  // (Abar - 1)/A
            if (any_tiny && tiny) coef = dt[k];                    // its limit at A = 0
            dbdd = a[k] * Bv[k];                                   // dBbar/ddelta
          } else {
            coef = dt[k];
            dbdd = Bv[k];
          }
          // ddelta: gh * (hprev * A * Abar + u * dBbar/ddelta)
          gdt[k] = __builtin_fmaf(P * hprev, An, gdt[k]);
          gdt[k] = __builtin_fmaf(gu, dbdd, gdt[k]);
          // dA: gh * hprev * delta * Abar + gh * u * dBbar/dA, where the ZOH
          // dBbar/dA = (delta*Abar*B - Bbar)/A (limit delta^2 B / 2 at A = 0)
          // (1/A is stored as 0 where A ~ 0, which drops the non-limit terms there)
          dA1[n] = __builtin_fmaf(dt[k], P * hprev, dA1[n]);
          if constexpr (ZOH) {
            dA1[n] = __builtin_fmaf(gu * dt[k], dbdd * ia, dA1[n]);
            dA2 = __builtin_fmaf(gh, beta[k], dA2);
            if (any_tiny && tiny) dA1[n] = __builtin_fmaf(gu, 0.5f * dt[k] * dt[k] * Bv[k], dA1[n]);
          }
          const float s = gh * coef;
          du[k] = __builtin_fmaf(s, Bv[k], du[k]);
          dBv[k] = active ? s * uv[k] : 0.0f;
          dCv[k] = active ? gy[k] * hv[k] : 0.0f;
          g = P;
        }
        if constexpr (ZOH) dA1[n] = __builtin_fmaf(-dA2, ia, dA1[n]);

        // ---- dB/dC: sum over the wave's 4 channels, then over the block ----
        float rb[2], rc[2];
        reduce_scatter_rows8(dBv, rb);
        reduce_scatter_rows8(dCv, rc);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int tt = j * K + 4 * m + row;
          atomicAdd(&acc[0][n][tt], rb[m]);
          atomicAdd(&acc[1][n][tt], rc[m]);
        }
      }
      mem_fence_compiler();
    }

    // ---- per-step outputs ----
    float ddl[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      ddl[k] = (k < nvalid) ? gdt[k] * sig[k] : 0.0f;
      db_acc += ddl[k];
    }
    if (active) {
      store_items<float, K>(p.du + c * L, tl, L, full, du);
      store_items<float, K>(p.ddelta + c * L, tl, L, full, ddl);
    }
    if (z_row) {
      float zv[K], dov[K], dzv[K];
      load_items<T, K>(z_row, tl, L, full, zv);
      load_items<T, K>(do_row, tl, L, full, dov);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float sg = sigmoid(zv[k]);
        dzv[k] = dov[k] * yv[k] * sg * __builtin_fmaf(zv[k], 1.0f - sg, 1.0f);
      }
      if (active) store_items<float, K>(p.dz + c * L, tl, L, full, dzv);
    }
    if (ch > 0) {
      if constexpr (TILE) stage.store(reinterpret_cast<float*>(tile_mem[buf ^ 1]), N, tid);
      store_states(buf ^ 1, hreg);
    }
    __syncthreads();
    // flush this chunk's dB/dC sums (all waves have added them) and clear
    for (int i = tid; i < 2 * NT * TCH; i += kBlock) {
      const int which = i / (NT * TCH);
      const int rest = i - which * NT * TCH;
      const int n = rest / TCH, tt = rest - n * TCH;
      float* slot = &acc[which][n][tt];
      const float v = *slot;
      *slot = 0.0f;
      const int64_t t = t0 + tt;
      if (n < N && t < L) unsafeAtomicAdd((which ? p.dC : p.dB) + (b * N + n) * L + t, v);
    }
    __syncthreads();
  }

  // ---- per-channel reductions over the channel's lanes ----
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (n < N) {
      const float s = group_sum<R>(dA1[n]);
      if (active && j == 0) unsafeAtomicAdd(p.dA + d * N + n, s);
      if (active && j == 0 && p.dh0) p.dh0[c * N + n] = gcarry[n];
    }
  }
  const float sD = group_sum<R>(dD_acc);
  const float sb = group_sum<R>(db_acc);
  if (active && j == 0) {
    if (p.dD) unsafeAtomicAdd(p.dD + d, sD);
    if (p.dbias) unsafeAtomicAdd(p.dbias + d, sb);
  }
}

// Clears the accumulated gradients (dA, dB, dC, dD, ddelta_bias) on the
// stream with a plain kernel (no hipMemsetAsync).
static __global__ __launch_bounds__(256) void bwd_zero_kernel(const BwdParams p) {
  const int64_t nbc = p.batch * p.N * p.L;
  const int64_t na = p.dim * p.N;
  const int64_t total = 2 * nbc + na + 2 * p.dim;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    if (i < nbc) p.dB[i] = 0.0f;
    else if (i < 2 * nbc) p.dC[i - nbc] = 0.0f;
    else if (i < 2 * nbc + na) p.dA[i - 2 * nbc] = 0.0f;
    else {
      const int64_t k = i - 2 * nbc - na;
      float* dst = k < p.dim ? p.dD : p.dbias;
      if (dst) dst[k < p.dim ? k : k - p.dim] = 0.0f;
    }
  }
}

template <typename T, int NT, bool ZOH, bool VEC>
static hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t nblocks = p.batch * p.groups;
  hipLaunchKernelGGL((scan_bwd_kernel<T, NT, ZOH, VEC>), dim3((unsigned)nblocks), dim3(kBlock), 0,
                     s, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_bwd_t(const BwdParams& p, int disc, bool vec, hipStream_t s) {
  {
    const int64_t total = 2 * p.batch * p.N * p.L + p.dim * p.N + 2 * p.dim;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool zoh = disc == 0;
  if (p.N <= 16) {
    if (zoh) return vec ? launch_bwd<T, 16, true, true>(p, s) : launch_bwd<T, 16, true, false>(p, s);
    return vec ? launch_bwd<T, 16, false, true>(p, s) : launch_bwd<T, 16, false, false>(p, s);
  }
  if (zoh) return vec ? launch_bwd<T, 64, true, true>(p, s) : launch_bwd<T, 64, true, false>(p, s);
  return vec ? launch_bwd<T, 64, false, true>(p, s) : launch_bwd<T, 64, false, false>(p, s);
}

}  // namespace mscan

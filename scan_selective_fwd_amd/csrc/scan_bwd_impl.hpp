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
// with the ZOH coefficient (Abar - 1)/A and its A-derivative
// dBbar/dA = B delta^2 psi(delta A) formed without cancellation
// (expm1_zoh, dcoef_dA in device_common.hpp).
//   dB_t[n] = sum_d gh_t u_t Bbar_t/B_t,  dC_t[n] = sum_d gy_t h_t[n]
//   dz_t    = dout_t y_t SiLU'(z_t),  dD = sum gy u,  ddelta_bias = sum ddelta
// With g_t = Abar_t gh_t the reverse recurrence is g_t = Abar_t (g_{t+1} + e_t),
// e_t = C_t gy_t: an affine map per step, so it scans like the forward, with
// suffix instead of prefix composition.
//
// Launches (api.cpp): a zero fill of the accumulated gradients; the forward
// kernel in states-only mode (the state at every chunk start, into the
// workspace); then this kernel.  Here a block serves 16 or 48 channels of one
// batch row (4 per wave, 16 lanes each, 8 steps per lane: 128-step chunks) and walks
// the chunks from last to first.  Per chunk and state index n it replays the
// forward from the stored chunk-start state (pass 1, DPP prefix scan, pass 2
// keeping h in registers), then the adjoint (reverse pass 1, DPP suffix scan
// with the carry from the later chunk, reverse pass 2) and the gradient
// terms.  The B/C chunk and the chunk-start states are staged in LDS once per
// block.  dB/dC are summed over the wave's 4 channels with gfx950 permlane
// swaps, over the block's waves through per-wave LDS slices (plain stores,
// summed after a barrier every 2 state indices), and into global memory with
// one float atomic per (n, t) per block.  dA, dD, ddelta_bias are summed over the
// channel's lanes and atomically over batch rows.  Atomics make the result
// deterministic only up to float32 rounding order.
//
// Long sequences with few channels are split into segments of whole chunks,
// one block per (batch row, segment, channel group).  The adjoint entering a
// segment from the right is then the composition of the later segments' affine
// maps (each an adjoint from a zero end plus a decay exp(A sum(delta))),
// carried by scan_bwd_seg.hip before this kernel; the chunk-start states come
// from a segmented forward pass.  Only segment 0 writes dh0.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_fwd_impl.hpp"
#include "tile_stage.hpp"

namespace mscan {

// Lane i receives lane i+1 of its 16-lane row; lane 15 receives `last`.
__device__ __forceinline__ float row_shift_left(float v, float last) {
  return dpp_mov<0x101 /*row_shl:1*/>(last, v);
}

// Moves between fixed lanes of every 16-lane row (other lanes: unspecified).
template <int k>   // lane k -> lane 0 (row_shl:k)
__device__ __forceinline__ float row_lane_to_first(float v) {
  if constexpr (k == 0) return v;
  else return dpp_mov<0x100 + k>(v, v);
}
template <int k>   // lane k -> lane 15 (row_shr:15-k)
__device__ __forceinline__ float row_lane_to_last(float v) {
  if constexpr (k == 15) return v;
  else return dpp_mov<0x110 + (15 - k)>(v, v);
}
template <int k>   // lane 0 -> lane k (row_shr:k)
__device__ __forceinline__ float row_first_to_lane(float v) {
  if constexpr (k == 0) return v;
  else return dpp_mov<0x110 + k>(v, v);
}
template <int k>   // lane 15 -> lane k (row_shl:15-k)
__device__ __forceinline__ float row_last_to_lane(float v) {
  if constexpr (k == 15) return v;
  else return dpp_mov<0x100 + (15 - k)>(v, v);
}

template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// TINY = false: the fast kernel, for blocks whose A are all negative.  A block
// in which some channel has A ~ 0 or A > 0 (ZOH only) sets its flag in
// p.deferred and exits without computing; the TINY = true kernel, launched
// right after on the same stream, computes exactly the flagged blocks, with
// the sign-agnostic ZOH coefficient and its A = 0 limit.
//
// Per-state values that live across state indices (the chunk-start state,
// the adjoint carried from the later chunk, the dA sum) are kept in
// registers "lane n holds state n": a channel's 16 lanes hold 16 states per
// register, and DPP row shifts bring state n to lane 0 or lane 15 and back.
//
// RST: packed sequences (p.reset flags).  The state entering a flagged step
// is zero: the step's decay factor in the recurrence and in the adjoint
// becomes 0 (Bbar keeps the true one), and its h_{t-1} counts as 0.
// NW: waves per block (4: 16 channels; 12: 48 channels, a whole CU at three
// waves per SIMD, whose dB/dC flushes sum three times as many channels before
// the global atomics).
template <typename T, int NT, bool ZOH, bool VEC, bool TINY, bool RST = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void scan_bwd_kernel(
    const BwdParams p) {
  constexpr int R = 16;
  constexpr int K = kItemsBwd;
  static_assert(K == 8, "the row reduce-scatter assumes 8 steps per lane");
  static_assert(NT % 16 == 0, "states are spread over the 16 lanes of a channel");
  constexpr int NTH = 64 * NW;   // threads per block
  constexpr int CPW = 64 / R;
  constexpr int CPB = NW * CPW;
  constexpr int TCH = R * K;
  constexpr bool TILE = (NT == 16);
  constexpr int NQ = NT / 16;
  // single-buffered: refilled between the two barriers that close a chunk
  __shared__ float4 tile_mem[TILE ? 2 * NT * TCH / 4 : 1];   // B, C rows of the chunk
  __shared__ float4 prm[CPB][NT];       // {A log2(e), 1/A (0 where A ~ 0), A, 1/A^2}
  // dB, dC partial sums of each wave for a group of G state indices, double
  // buffered: written with plain stores, summed over the waves and flushed
  // to global memory after the group's barrier.  (LDS float atomics are far
  // slower than stores on this chip.)  Step tt of the chunk sits at
  // position (tt % 8) * 16 + tt / 8, which makes each wave's 64 stores hit
  // 64 consecutive words.
  constexpr int G = 2;
  __shared__ float red[2][NW][2][G][TCH];
  // per-step factors of the epilogue, made when the inputs are first read
  // (softplus'(r) for ddelta and dout*SiLU'(z) for dz), so that the inputs
  // are not read from memory a second time; [k][tid] keeps accesses
  // conflict-free
  __shared__ float stash[2][kItemsBwd][NTH];

  // the TINY launch computes only the blocks the fast launch deferred; the
  // others leave before loading anything
  if constexpr (ZOH && TINY) {
    if (p.deferred[blockIdx.x] == 0) return;   // block-uniform
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane % R;
  const int row = lane / R;
  const int cl = wave * CPW + row;
  // block order (b, segment, group) with the group fastest, as in the forward
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t ngrp = (p.dim + CPB - 1) / CPB;   // this kernel's channel groups per batch row
  const int64_t per_b = ngrp * p.nseg;
  const int64_t b = blk / per_b;
  const int64_t seg = (blk - b * per_b) / ngrp;
  const int64_t grp = blk - b * per_b - seg * ngrp;
  const int64_t d_raw = grp * CPB + cl;
  const bool active = d_raw < p.dim;
  const int64_t d = active ? d_raw : p.dim - 1;
  const int64_t c = b * p.dim + d;
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t nchunks = p.nchunks;
  const int64_t ch_begin = p.seg_chunks > 0 ? seg * p.seg_chunks : 0;
  const int64_t ch_end =
      p.seg_chunks > 0 ? (ch_begin + p.seg_chunks < nchunks ? ch_begin + p.seg_chunks : nchunks)
                       : nchunks;

  // this lane's channel row as block-uniform base + lane part; the row
  // addresses are formed from an opaque copy of the lane part where they are
  // used, so that none is kept (and spilled) across the chunk loop
  const int64_t c_blk = b * p.dim + grp * CPB;
  const int cl_eff = (int)(d - grp * CPB);
  const T* __restrict__ B_b = static_cast<const T*>(p.B) + b * N * L;
  const T* __restrict__ C_b = static_cast<const T*>(p.C) + b * N * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const uint8_t* __restrict__ rst_row = RST ? p.reset + b * L : nullptr;

  bool my_tiny = false;
  for (int i = tid; i < CPB * NT; i += NTH) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    const bool real = dd < p.dim && n < N;
    const float a = real ? p.A[dd * N + n] : -1.0f;
    const bool tiny = __builtin_fabsf(a) < 1e-30f;
    // blocks with any A that is not strictly negative (A ~ 0, A > 0) are
    // deferred to the TINY launch, which forms the coefficient generally
    my_tiny |= real && !(a < -1e-30f);
    prm[ci][n] = make_float4(a * kLog2e, tiny ? 0.0f : 1.0f / a, a, tiny ? 0.0f : 1.0f / (a * a));
  }

  // chunk-start states of this lane's channel: lane j holds state 16 q + j
  auto load_states = [&](int64_t ch, float (&dst)[NQ]) {
    const float* __restrict__ st_row =
        p.chunk_states + (c_blk + opaque_int(cl_eff)) * nchunks * N;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int n = 16 * q + j;
      dst[q] = (active && n < N) ? st_row[ch * N + n] : 0.0f;
    }
  };

  TileStager<T, TCH, K, NT, TILE ? 2 * NT : 1, NTH> stage;
  float hreg[NQ], gcreg[NQ], dAreg[NQ];
  // the adjoint entering the block's last chunk from the right: zero at the
  // end of the sequence (no gradient flows into the final state), else the
  // carry over the later segments
  const float* gin = p.seg_gin ? p.seg_gin + (c * p.nseg + seg) * N : nullptr;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int n = 16 * q + j;
    gcreg[q] = (gin && active && n < N) ? gin[n] : 0.0f;
    dAreg[q] = 0.0f;
  }
  {
    const int64_t last = ch_end - 1;
    const bool full_last = VEC && last * TCH + TCH <= L;
    if constexpr (TILE) {
      stage.load(B_b, C_b, N, L, last * TCH, full_last, opaque_int(tid));
      stage.store(reinterpret_cast<float*>(tile_mem), N, opaque_int(tid));
    }
    load_states(last, hreg);
  }
  // barrier for the LDS fills; also: does any channel of the block have A ~ 0?
  const bool any_tiny = __syncthreads_or(my_tiny);
  if constexpr (ZOH) {
    if constexpr (!TINY) {
      if (tid == 0) p.deferred[blockIdx.x] = any_tiny ? 1 : 0;
      if (any_tiny) return;            // block-uniform: the TINY kernel takes it
    }
  }

  float dD_acc = 0.0f, db_acc = 0.0f;

  for (int64_t ch = ch_end - 1; ch >= ch_begin; --ch) {
    const int64_t t0 = ch * TCH;
    const int64_t tl = t0 + (int64_t)j * K;
    const bool full = VEC && t0 + TCH <= L;
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    float uv[K], dt[K], gy[K], yv[K], du[K], gdt[K];
    {
      const int64_t co = (c_blk + opaque_int(cl_eff)) * L;
      const T* __restrict__ u_row = static_cast<const T*>(p.u) + co;
      const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + co;
      const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + co : nullptr;
      const T* __restrict__ do_row = static_cast<const T*>(p.dout) + co;
      float raw[K], dov[K];
      load_items<T, K>(u_row, tl, L, full, uv);
      load_items<T, K>(dl_row, tl, L, full, raw);
      load_items<T, K>(do_row, tl, L, full, dov);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float r = raw[k] + bias;
        const float s = p.softplus ? softplus(r) : r;
        dt[k] = (k < nvalid) ? s : 0.0f;
        gy[k] = dov[k];
        stash[0][k][tid] = p.softplus ? sigmoid(r) : 1.0f;   // softplus'
      }
      if (z_row) {
        float zv[K];
        load_items<T, K>(z_row, tl, L, full, zv);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float sg = sigmoid(zv[k]);
          gy[k] *= zv[k] * sg;                                        // dout * SiLU(z)
          stash[1][k][tid] = dov[k] * sg * __builtin_fmaf(zv[k], 1.0f - sg, 1.0f);   // dz / y
        }
      }
    }
    float dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      // a channel slot past `dim` contributes nothing to the reduced gradients
      uv[k] = active ? uv[k] : 0.0f;
      gy[k] = active ? gy[k] : 0.0f;
      dsum += dt[k];
      yv[k] = Dd * uv[k];
      du[k] = Dd * gy[k];
      gdt[k] = 0.0f;
      dD_acc = __builtin_fmaf(gy[k], uv[k], dD_acc);
    }
    float keep[K];
    float lane_keep = 1.0f;
    if constexpr (RST) lane_keep = load_keep<K>(rst_row, tl, L, keep) ? 0.0f : 1.0f;

    const float* tB = reinterpret_cast<const float*>(tile_mem);
    float4 pr_next = prm[cl][0];
    // state indices in groups of 16 (the 16 lanes of a channel hold one
    // group's per-state registers); N <= 16 is a single group
    for (int q = 0; q < NQ; ++q) {
     float hq = hreg[q], gq = gcreg[q], dq = dAreg[q];
     static_for<0, 16>([&](auto nc) {
      constexpr int nl = decltype(nc)::value;
      const int n = q * 16 + nl;
      const float4 pr = pr_next;
      if (n + 1 < NT) pr_next = prm[cl][n + 1];
      if (n < N) {
        const float a2 = pr.x, ia = pr.y, An = pr.z, iA2 = pr.w;
        const float h_in = row_lane_to_first<nl>(hq);   // state n, in lane 0
        const float gc = row_lane_to_last<nl>(gq);      // carry n, in lane 15
        float Bv[K], Cv[K];
        auto read_bc = [&]() {
          if constexpr (TILE) {
            tile_read<K>(tB + n * TCH, j, Bv);
            tile_read<K>(tB + (NT + n) * TCH, j, Cv);
          } else {
            load_items<T, K>(B_b + (int64_t)n * L, tl, L, full, Bv);
            load_items<T, K>(C_b + (int64_t)n * L, tl, L, full, Cv);
          }
        };
        read_bc();
        // TINY: where A ~ 0 (1/A stored as 0) the ZOH coefficient
        // (e^{dA}-1)/A takes its limit delta
        const bool tiny = TINY && ia == 0.0f;

        // ---- replay, pass 1: each lane's steps folded into its summary ----
        // coef[k] is the ZOH coefficient (Abar - 1)/A (its limit delta at
        // A = 0; delta under Euler); Bbar u = coef B u is formed again where
        // it is used, which keeps one array fewer live across the scans
        float a[K], coef[K], ghv[K];
        float agg;
        // a step's decay in the recurrence and the adjoint (0 at a flagged step)
        auto decay = [&](int k) { return RST ? a[k] * keep[k] : a[k]; };
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float z = dt[k] * a2;
          a[k] = fast_exp2(z);
          if constexpr (ZOH && !TINY) {
            coef[k] = zoh_coef_neg(dt[k], z, a[k], ia, ia * -kCoefBound);   // A < 0 here
          } else if constexpr (ZOH) {
            coef[k] = tiny ? dt[k] : expm1_zoh(z, a[k]) * ia;
          } else {
            coef[k] = dt[k];
          }
          const float beta = coef[k] * (Bv[k] * uv[k]);
          agg = k == 0 ? beta : __builtin_fmaf(decay(k), agg, beta);
        }
        const float Alane = RST ? fast_exp2(a2 * dsum) * lane_keep : fast_exp2(a2 * dsum);
        float Ag = Alane;
        agg = (j == 0) ? __builtin_fmaf(Ag, h_in, agg) : agg;   // chunk-start state enters lane 0

        // ---- adjoint, pass 1: g_t = Abar_t (g_{t+1} + C_t gy_t) folded ----
        float gagg = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) gagg = decay(k) * __builtin_fmaf(Cv[k], gy[k], gagg);
        float As = Alane;
        gagg = (j == R - 1) ? __builtin_fmaf(As, gc, gagg) : gagg;   // later chunk enters lane 15

        // the replay's prefix scan and the adjoint's suffix scan together
        dual_scan_row_fused(Ag, agg, As, gagg);
        const float hstart = group_shift_right<R>(agg, h_in);   // state before this lane's steps
        float g = row_shift_left(gagg, gc);                 // adjoint entering each lane from the right
        const float gc_new = row_first_to_lane<nl>(gagg);   // leaving lane 0, now in lane n
        gq = (j == nl) ? gc_new : gq;

        // ---- adjoint, pass 2: dL/dh_t of each step ----
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
          ghv[k] = __builtin_fmaf(Cv[k], gy[k], g);
          g = decay(k) * ghv[k];
        }

        // B and C again from the tile (LDS): kept from the first reads, their
        // registers would be live across the scans (the fence keeps the
        // compiler from reusing those reads)
        if constexpr (TILE) {
          mem_fence_compiler();
          read_bc();
        }
        // ---- replay, pass 2, with the gradient terms: dB/dC are summed
        //      over the wave's 4 channels as soon as each pair of steps is
        //      done; dA collects delta P h_{t-1} (the Abar path) and, under
        //      ZOH, dcoef/dA gh B u (the Bbar path), with no division by A ----
        float dAp = 0.0f;
        float pB = 0.0f, pC = 0.0f, sB[4], sC[4], TB[2], TC[2];
        float h = hstart;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float Bu = Bv[k] * uv[k];
          const float hprev = RST ? h * keep[k] : h;
          const float hk = __builtin_fmaf(decay(k), h, coef[k] * Bu);
          yv[k] = __builtin_fmaf(Cv[k], hk, yv[k]);
          const float gh = ghv[k];                           // dL/dh_t
          const float P = gh * a[k];
          if constexpr (ZOH) {
            // ddelta: gh Abar (A h_{t-1} + B u), since dBbar/ddelta = Abar B
            gdt[k] = __builtin_fmaf(P, __builtin_fmaf(An, hprev, Bu), gdt[k]);
            const float zeta = dcoef_dA(dt[k] * a2, a[k], dt[k] * dt[k], iA2);
            dAp = __builtin_fmaf(dt[k] * P, hprev, __builtin_fmaf(zeta, gh * Bu, dAp));
          } else {
            // Euler: Bbar = delta B, no A dependence
            gdt[k] = __builtin_fmaf(P * An, hprev, __builtin_fmaf(gh, Bu, gdt[k]));
            dAp = __builtin_fmaf(dt[k] * P, hprev, dAp);
          }
          const float s = gh * coef[k];
          du[k] = __builtin_fmaf(s, Bv[k], du[k]);
          const float vB = s * uv[k];
          const float vC = gy[k] * hk;
          if (!(k & 1)) {
            pB = vB;
            pC = vC;
          } else {
            sB[k / 2] = rs_pair16(pB, vB);
            sC[k / 2] = rs_pair16(pC, vC);
            if (k == 3) {
              TB[0] = rs_pair32(sB[0], sB[1]);
              TC[0] = rs_pair32(sC[0], sC[1]);
            } else if (k == 7) {
              TB[1] = rs_pair32(sB[2], sB[3]);
              TC[1] = rs_pair32(sC[2], sC[3]);
            }
          }
          h = hk;
        }
        const int buf = (n / G) & 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) {   // lane (row r, j) owns step j*K + 4m + r
          const int pos = (4 * m + row) * 16 + j;
          red[buf][wave][0][n % G][pos] = TB[m];
          red[buf][wave][1][n % G][pos] = TC[m];
        }
        const float dAn = row_last_to_lane<nl>(row_sum_to_last(dAp));
        dq += (j == nl) ? dAn : 0.0f;
      }
      if constexpr (nl % G == G - 1) {
        // end of a group of G states: sum the waves' partials and add them
        // to dB, dC (block-uniform condition: N is the same for all threads)
        const int n0 = n - (G - 1);
        const int buf = (n / G) & 1;
        if (n0 < N) {
          __syncthreads();
          // (the thread index is hidden from the optimizer: the atomics'
          // addresses derived from it were otherwise formed once, before the
          // chunk loop, and spilled -- their reloads read scratch from HBM)
#pragma unroll 1
          for (int i = opaque_int(tid); i < 2 * G * TCH; i += NTH) {
            const int which = i / (G * TCH);
            const int nn = (i / TCH) % G;
            // consecutive threads take consecutive steps, so that each wave's
            // global atomics cover the fewest cache lines
            const int tt = i % TCH;
            const int pos = (tt % K) * 16 + tt / K;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[buf][w][which][nn][pos];
            if (n0 + nn < N && t0 + tt < L)
              unsafeAtomicAdd((which ? p.dC : p.dB) + (b * N + n0 + nn) * L + t0 + tt, v);
          }
        }
      }
      mem_fence_compiler();
     });
     gcreg[q] = gq;
     dAreg[q] = dq;
    }

    // the earlier chunk's B/C rows and states: issued here (not at the chunk
    // start) so their registers are not live across the state-index loop
    if (ch > ch_begin) {
      if constexpr (TILE)   // earlier chunks are full
        stage.load(B_b, C_b, N, L, t0 - TCH, VEC, opaque_int(tid));
      load_states(ch - 1, hreg);
    }

    // ---- per-step outputs ----
    const int64_t co = (c_blk + opaque_int(cl_eff)) * L;
    {
      float ddl[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        ddl[k] = (k < nvalid) ? gdt[k] * stash[0][k][tid] : 0.0f;
        db_acc += ddl[k];
      }
      if (active) {
        store_items<float, K>(p.du + co, tl, L, full, du);
        store_items<float, K>(p.ddelta + co, tl, L, full, ddl);
      }
    }
    if (p.z) {
      float dzv[K];
#pragma unroll
      for (int k = 0; k < K; ++k) dzv[k] = yv[k] * stash[1][k][tid];
      if (active) store_items<float, K>(p.dz + co, tl, L, full, dzv);
    }
    // every wave is past the last group barrier, so no wave still reads the
    // tile: refill it with the earlier chunk.  The barrier also keeps the
    // next chunk's slice stores behind this chunk's last flush.
    if (ch > ch_begin) {
      if constexpr (TILE) stage.store(reinterpret_cast<float*>(tile_mem), N, opaque_int(tid));
      __syncthreads();
    }
  }

  // ---- per-channel results: dh0, dA (over batch rows), dD, ddelta_bias ----
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int n = 16 * q + j;
    if (active && n < N) {
      if (p.dh0 && seg == 0) p.dh0[c * N + n] = gcreg[q];
      unsafeAtomicAdd(p.dA + d * N + n, dAreg[q]);
    }
  }
  const float sD = row_sum_to_last(dD_acc);
  const float sb = row_sum_to_last(db_acc);
  if (active && j == R - 1) {
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

template <typename T, int NT, bool ZOH, bool VEC, bool RST, int NW>
static hipError_t launch_bwd_x(const BwdParams& p, hipStream_t s, hipEvent_t ev_begin,
                               hipEvent_t ev_end) {
  const int64_t nblocks = p.batch * ((p.dim + 4 * NW - 1) / (4 * NW)) * p.nseg;
  hipError_t e;
  if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
  hipLaunchKernelGGL((scan_bwd_kernel<T, NT, ZOH, VEC, false, RST, NW>),
                     dim3((unsigned)nblocks), dim3(64 * NW), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
  if (!ZOH) return e;
  hipLaunchKernelGGL((scan_bwd_kernel<T, NT, ZOH, VEC, true, RST, NW>),
                     dim3((unsigned)nblocks), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

// N <= 16 without reset flags, in one pass, takes 12-wave blocks when they
// number at least kBwdWideMinBlocks, else 4-wave blocks.  Measured (f32
// batch 8, D 1536, L 2048: 256 wide blocks): 0.652-0.662 ms against 0.682 ms,
// with a third of the dB/dC atomics; bf16 batch 2, D 5120 (214 wide blocks,
// 640 narrow): 0.622-0.629 ms against 0.682-0.685 ms.  Segmented (bf16
// batch 1, D 1024, 32 segments from L = 4096): narrow blocks 7-12 % faster.
template <typename T, int NT, bool ZOH, bool VEC, bool RST>
static hipError_t launch_bwd(const BwdParams& p, hipStream_t s, hipEvent_t ev_begin,
                             hipEvent_t ev_end) {
  if constexpr (NT == 16 && !RST) {
    if (p.nseg == 1 && p.batch * ((p.dim + 47) / 48) >= kBwdWideMinBlocks)
      return launch_bwd_x<T, NT, ZOH, VEC, RST, 12>(p, s, ev_begin, ev_end);
  }
  return launch_bwd_x<T, NT, ZOH, VEC, RST, 4>(p, s, ev_begin, ev_end);
}

// The backward for one state-size variant (NT = 16: N <= 16; NT = 64: N <= 64):
// the zero fill, then the kernel for the discretization and load width.
// Each variant is compiled in a translation unit of its own.
template <typename T, int NT, bool RST>
static hipError_t dispatch_bwd_nt(const BwdParams& p, int disc, bool vec, hipStream_t s,
                                  hipEvent_t ev_begin, hipEvent_t ev_end) {
  {
    const int64_t total = 2 * p.batch * p.N * p.L + p.dim * p.N + 2 * p.dim;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 1024) blocks = 1024;   // grid-stride: a few elements per thread
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const hipEvent_t b = ev_begin, e = ev_end;
  if (disc == 0)
    return vec ? launch_bwd<T, NT, true, true, RST>(p, s, b, e)
               : launch_bwd<T, NT, true, false, RST>(p, s, b, e);
  return vec ? launch_bwd<T, NT, false, true, RST>(p, s, b, e)
             : launch_bwd<T, NT, false, false, RST>(p, s, b, e);
}

}  // namespace mscan

// Fused selective-scan forward for gfx950 (kernel template; instantiated per
// element type in scan_fwd_{f32,bf16}.hip and, in states-only mode, in
// scan_states_{f32,bf16}.hip).
//
// What is computed (chapterpal.com page on the Mamba paper, Knowl 1
// "Selective State Space Layer (S6)", steps 3-4, with diagonal A):
//   Abar_t = exp(delta_t A), Bbar_t = (exp(delta_t A) - 1)/A * B_t  (ZOH)
//   h_t = Abar_t h_{t-1} + Bbar_t u_t,  y_t = C_t . h_t
// plus the library's additions y += D u, out = y * SiLU(z), Euler Bbar.
//
// How (MI355X-first; the pages' fused-kernel outline -- load the parameters
// once, discretize and scan on chip, write only y -- is the paper-graph-ui
// summary's section 3.4 "Kernel fusion" and its chunking paragraph):
//   * A block serves CPB channels of ONE batch row; a channel (b, d) owns R
//     lanes of a wave and lane j owns K consecutive steps of each chunk of
//     R*K steps.  u, delta, z are read once per lane with 16-byte loads; the
//     B and C chunk, shared by all the block's channels, is staged once per
//     block into an LDS tile (tile_stage.hpp); out is written once.  The
//     expanded (B, L, D, N) Abar/Bbar/h never leave registers.
//   * Per state index n: pass 1 discretizes the lane's K steps in registers
//     (one v_exp_f32 per step) and folds them into the lane's affine summary
//     (A_lane, B_lane); A_lane is exp(A * sum(delta)), one exponential per
//     lane instead of K multiplies.  A DPP scan over the channel's R lanes
//     (fused v_fmac/v_mul with row_shr / row_bcast sources, no LDS) turns the
//     summaries into each lane's starting state, composed with the state
//     carried in from the previous chunk.  Pass 2 replays the K steps from
//     that state and accumulates y_t += C_t[n] h_t[n].
//   * Chunks follow each other inside the block; the carried state is a
//     register per n (the pages' "chunk boundary" carry).  The next chunk's
//     u/delta and B/C loads are in flight while the current one computes.
// No atomics, no workspace: the result is bitwise deterministic.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_stage.hpp"

#include <type_traits>

namespace mscan {

// K elements of a row from step t: vector loads when `full` (the whole
// chunk lies inside the sequence and rows are 16-byte aligned), else
// element loads with steps past L reading 0.
template <typename T, int K>
__device__ __forceinline__ void load_items(const T* __restrict__ row, int64_t t, int64_t L,
                                           bool full, float (&v)[K]) {
  if (full) {
    Elem<T>::template load_k<K>(row + t, v);
  } else {
    const int64_t rem = L - t;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    Elem<T>::template load_k_guarded<K>(row + t, nvalid, v);
  }
}

// Reset flags of a lane's K steps: keep[k] = 0 where the state is zeroed
// before step tl + k, else 1 (steps past L keep it).  Returns whether any
// flag is set.
template <int K>
__device__ __forceinline__ bool load_keep(const uint8_t* __restrict__ row, int64_t tl, int64_t L,
                                          float (&keep)[K]) {
  bool any = false;
  if (K % 8 == 0 && tl + K <= L && (reinterpret_cast<uintptr_t>(row + tl) & 7) == 0) {
    // the lane's flags with 8-byte loads
#pragma unroll
    for (int i = 0; i < K / 8; ++i) {
      const uint2 v = *reinterpret_cast<const uint2*>(row + tl + 8 * i);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool r = (((k < 4 ? v.x : v.y) >> (8 * (k & 3))) & 0xFFu) != 0u;
        keep[8 * i + k] = r ? 0.0f : 1.0f;
        any |= r;
      }
    }
    return any;
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t t = tl + k;
    const bool r = t < L && row[t] != 0;
    keep[k] = r ? 0.0f : 1.0f;
    any |= r;
  }
  return any;
}

template <typename T, int K>
__device__ __forceinline__ void store_items(T* __restrict__ row, int64_t t, int64_t L, bool full,
                                            const float (&v)[K]) {
  if (full) {
    Elem<T>::template store_k<K>(row + t, v);
  } else {
    const int64_t rem = L - t;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    if (nvalid > 0) Elem<T>::template store_k_guarded<K>(row + t, nvalid, v);
  }
}

// MODE (FwdMode): kModeOut computes the outputs (and, when p.chunk_states is
// set, also saves the state at the start of every chunk as checkpoints for
// the backward).  kModeChunkStates is the backward's recompute pass: it only
// writes the state at the start of every chunk (to p.chunk_states).
// kModeSegSummary runs each segment of a long sequence from a zero state and
// writes its end state and delta sum.  The two state-only modes skip C, z, y
// and out.
//
// A block serves one channel group of one batch row, for the whole sequence
// or (p.seg_chunks > 0) for one segment of it.  A segmented run takes three
// launches, in one of two schemes (the carry kernel in the middle composes
// the segments' end states from zero into the state entering each segment,
// p.seg_h0):
//  * short segments: the summary mode, the carry, then SEG = kSegWhole runs
//    every segment from p.seg_h0;
//  * long segments: SEG = kSegLocal runs every segment from a zero state and
//    also writes the summaries, the carry, then SEG = kSegFix runs each
//    segment again from its entering state over its first chunks only.  The
//    true state is the zero-start state plus exp(A * sum(delta)) times the
//    entering state; kSegFix stops once that second term is below 2^-160 for
//    every (channel, n) of the block, or a reset flag has cut it, and from
//    there on the first launch's outputs and checkpoints stand.  This saves
//    the summary pass (about 0.65 of an output pass) at the price of the
//    chunks the entering state takes to decay.
//
// RST: packed sequences.  Where p.reset flags a step the state entering it is
// zero: the step's decay factor in the recurrence (not in Bbar) becomes 0,
// and so does the decay of any lane summary that contains the step.
//
// EXACT: N == NT, known at compile time.  The unrolled loop over state
// indices then has no per-index branch, and the operands of index n + 1
// need no copies at the join of one (a fifth fewer VALU instructions).
template <typename T, int R, int K, int NT, bool ZOH, bool VEC, int MODE, bool RST = false,
          bool EXACT = false, int SEG = kSegWhole>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void scan_fwd_kernel(
    const FwdParams p) {
  constexpr bool STATES = MODE != kModeOut;
  constexpr bool FIX = SEG == kSegFix;
  constexpr bool LOCAL = SEG == kSegLocal;   // every segment from zero, summaries written
  constexpr int CPW = 64 / R;   // channels per wave
  constexpr int CPB = (kBlock / 64) * CPW;
  constexpr int TCH = R * K;    // steps per chunk
  constexpr int TROWS = STATES ? NT : 2 * NT;
  // The LDS tile holds two chunks of B/C rows (2 * TROWS * TCH floats): it is
  // used for R = 16, N <= 16 (32 KB at K = 8); wider lane groups or larger N
  // read B/C per lane from global memory (L1/L2 cached) instead.
  constexpr bool TILE = (R == 16 && NT == 16);
  __shared__ float4 tile_mem[2][TILE ? TROWS * TCH / 4 : 1];
  __shared__ float a2s[CPB][NT], ias[CPB][NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane % R;
  const int cl = wave * CPW + lane / R;       // channel slot in the block
  // block order (b, segment, group) with the group fastest: consecutive
  // blocks share the B/C rows of one segment
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_b = p.groups * p.nseg;
  const int64_t b = blk / per_b;
  const int64_t seg = (blk - b * per_b) / p.groups;
  const int64_t grp = blk - b * per_b - seg * p.groups;
  const int64_t d_raw = grp * CPB + cl;
  const bool active = d_raw < p.dim;
  const int64_t d = active ? d_raw : p.dim - 1;
  const int64_t c = b * p.dim + d;
  const int N = EXACT ? NT : p.N;
  const int64_t L = p.L;

  // OPQ (reset flags, whose extra registers made the kernel spill most):
  // per-thread addresses are formed again in every chunk from an opaque lane
  // index instead of being kept across the chunk loop.  Without reset flags
  // keeping them measured faster.
  constexpr bool OPQ = RST;
  const int64_t c_blk = b * p.dim + grp * CPB;
  const int cl_eff = (int)(d - grp * CPB);
  auto lane_row = [&]() -> int64_t {
    return OPQ ? (c_blk + opaque_int(cl_eff)) * L : c * L;
  };
  auto tid_o = [&]() { return OPQ ? opaque_int(tid) : tid; };
  const T* __restrict__ u_row = static_cast<const T*>(p.u) + c * L;
  const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + c * L;
  const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + c * L : nullptr;
  T* __restrict__ out_row = static_cast<T*>(p.out) + c * L;
  const T* __restrict__ B_b = static_cast<const T*>(p.B) + b * N * L;
  const T* __restrict__ C_b = static_cast<const T*>(p.C) + b * N * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const uint8_t* __restrict__ rst_row = RST ? p.reset + b * L : nullptr;

  // per-channel constants: A * log2(e) and 1/A (0 where A is ~0, the ZOH limit)
  bool my_tiny = false;
  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    const bool real = dd < p.dim && n < N;
    const float a = real ? p.A[dd * N + n] : -1.0f;
    const bool tiny = __builtin_fabsf(a) < 1e-30f;
    // blocks with any A that is not strictly negative (A ~ 0, A > 0) take
    // the general copy of the chunk loop
    my_tiny |= real && !(a < -1e-30f);
    a2s[ci][n] = a * kLog2e;
    ias[ci][n] = tiny ? 0.0f : 1.0f / a;
  }

  // Carried state per n.  Only the FIRST lane of each channel's group holds
  // it (it is folded into that lane's summary before the scan).
  const int64_t nchunks = (L + TCH - 1) / TCH;
  const int64_t ch_begin = p.seg_chunks > 0 ? seg * p.seg_chunks : 0;
  const int64_t ch_end =
      p.seg_chunks > 0 ? (ch_begin + p.seg_chunks < nchunks ? ch_begin + p.seg_chunks : nchunks)
                       : nchunks;
  const float* h_enter = nullptr;
  if constexpr (FIX) h_enter = p.seg_h0 + (c * p.nseg + seg) * N;
  else if constexpr (!LOCAL && MODE != kModeSegSummary)
    h_enter = p.seg_h0 ? p.seg_h0 + (c * p.nseg + seg) * N : (p.h0 ? p.h0 + c * N : nullptr);
  float cr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) cr[n] = (n < N && h_enter) ? h_enter[n] : 0.0f;

  TileStager<T, TCH, K, NT, TILE ? TROWS : 1, kBlock> stage;
  float nu[K], nd[K];
  {
    const int64_t tb = ch_begin * TCH;
    const bool full0 = VEC && tb + TCH <= L;
    if constexpr (TILE) {
      stage.load(B_b, C_b, N, L, tb, full0, tid);
      stage.store(reinterpret_cast<float*>(tile_mem[0]), N, tid);
    }
    load_items<T, K>(u_row, tb + (int64_t)j * K, L, full0, nu);
    load_items<T, K>(dl_row, tb + (int64_t)j * K, L, full0, nd);
  }
  // The state entering each chunk: the backward's recompute pass, or
  // checkpoints a forward may save for a later backward (same 128-step
  // chunks: 16 lanes x 8 steps).  The first chunk's is stored here, the
  // others at the end of the chunk before them, where few registers are live.
  constexpr bool kCkpt = R == 16 && R * K == 16 * kItemsBwd;
  const bool save_states =
      MODE == kModeChunkStates || (MODE == kModeOut && kCkpt && p.chunk_states != nullptr);
  auto store_state = [&](int64_t ch) {
    if (save_states && active && j == 0) {
      float* dst = p.chunk_states + (c * nchunks + ch) * N;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        if (n < N) dst[n] = cr[n];
    }
  };
  store_state(ch_begin);
  float dtot = 0.0f;   // this lane's delta sum over the block's chunks
  bool seg_reset = false;   // RST: a flag in this lane's steps of the block
  // barrier for the LDS fills; also: does any channel of the block have A ~ 0?
  const bool any_tiny = __syncthreads_or(my_tiny);

  // TP: some channel of the block has A ~ 0 (ZOH; block-uniform): the chunk
  // loop is compiled twice, and only the copy such blocks run tests for the
  // limit of the ZOH coefficient.
  auto run_chunks = [&](auto tp_c) {
    constexpr bool TP = decltype(tp_c)::value;
    for (int64_t ch = ch_begin; ch < ch_end; ++ch) {
      if constexpr (FIX) {
        // what is left of the entering state: |h_enter[n]| exp(A_n sum(delta)),
        // in log2 so that a large entering state is not lost to underflow
        const float S = group_sum<R>(dtot);
        const bool cut = RST && group_sum<R>(seg_reset ? 1.0f : 0.0f) > 0.0f;
        bool alive = false;
        if (active && !cut)
          for (int n = 0; n < N; ++n)
            alive |= __builtin_fmaf(a2s[cl][n], S,
                                    __builtin_amdgcn_logf(__builtin_fabsf(h_enter[n]))) > -160.0f;
        if (!__syncthreads_or(alive)) break;   // block-uniform
      }
      const int buf = (int)((ch - ch_begin) & 1);
      const int64_t t0 = ch * TCH;
      const int64_t tl = t0 + (int64_t)(OPQ ? opaque_int(j) : j) * K;   // this lane's first step
      const bool full = VEC && t0 + TCH <= L;
      const bool more = ch + 1 < ch_end;
      const bool full_next = VEC && t0 + 2 * TCH <= L;
      const int64_t rem = L - tl;
      const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
      if constexpr (TILE) {
        if (more) stage.load(B_b, C_b, N, L, t0 + TCH, full_next, tid_o());
      }
      const T* __restrict__ u_c = OPQ ? static_cast<const T*>(p.u) + lane_row() : u_row;
      const T* __restrict__ dl_c = OPQ ? static_cast<const T*>(p.delta) + lane_row() : dl_row;

      float uv[K], dt[K], y[K], zv[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        uv[k] = nu[k];
        dt[k] = nd[k];
      }
      if (more) {
        load_items<T, K>(u_c, tl + TCH, L, full_next, nu);
        load_items<T, K>(dl_c, tl + TCH, L, full_next, nd);
      }
      if constexpr (!STATES) {
        if constexpr (OPQ) {
          if (p.z) load_items<T, K>(static_cast<const T*>(p.z) + lane_row(), tl, L, full, zv);
        } else {
          if (z_row) load_items<T, K>(z_row, tl, L, full, zv);
        }
      }
      float dsum = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float r = dt[k] + bias;
        float s = p.softplus ? softplus(r) : r;
        s = (k < nvalid) ? s : 0.0f;     // steps past L are the identity map
        dt[k] = s;
        dsum += s;
        y[k] = Dd * uv[k];
        if constexpr (!ZOH) uv[k] = s * uv[k];   // Euler: Bbar u = B (delta u)
      }
      dtot += dsum;
      float keep[K];
      float lane_keep = 1.0f;
      if constexpr (RST) {
        const bool any = load_keep<K>(rst_row, tl, L, keep);
        lane_keep = any ? 0.0f : 1.0f;
        seg_reset |= any;
      }

      const float* tB = reinterpret_cast<const float*>(tile_mem[buf]);
      // operands of state index n + 1 are read while n is computed
      // B of state index n + 1 is read while n is computed; C of n is read
      // at the start of n (it is first needed after pass 1 and the scan)
      float a2n = a2s[cl][0], ian = ias[cl][0];
      float Bn[K];
      if constexpr (TILE) tile_read<K>(tB, j, Bn);
      else load_items<T, K>(B_b, tl, L, full, Bn);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n < N) {
          const float a2 = a2n, ia = ian;
          float Bv[K], Cv[K];
#pragma unroll
          for (int k = 0; k < K; ++k) Bv[k] = Bn[k];
          if constexpr (!STATES) {
            if constexpr (TILE) tile_read<K>(tB + (NT + n) * TCH, j, Cv);
            else load_items<T, K>(C_b + (int64_t)n * L, tl, L, full, Cv);
          }
          if (n + 1 < N) {
            a2n = a2s[cl][n + 1];
            ian = ias[cl][n + 1];
            if constexpr (TILE) tile_read<K>(tB + (n + 1) * TCH, j, Bn);
            else load_items<T, K>(B_b + (int64_t)(n + 1) * L, tl, L, full, Bn);
          }
          float a[K], beta[K];
          float agg = 0.0f;
          if constexpr (!TP) {
            // every A of the block is negative here
            const float mb = ia * -kCoefBound;
#pragma unroll
            for (int k = 0; k < K; ++k) {
              const float z = dt[k] * a2;
              a[k] = fast_exp2(z);
              if constexpr (ZOH) {
                // (Abar - 1)/A * B * u
                beta[k] = zoh_coef_neg(dt[k], z, a[k], ia, mb) * (Bv[k] * uv[k]);
              } else {
                beta[k] = Bv[k] * uv[k];
              }
              if constexpr (RST) a[k] *= keep[k];
              agg = k == 0 ? beta[0] : __builtin_fmaf(a[k], agg, beta[k]);
            }
          } else {
            // a channel of this block has A ~ 0 (stored as 1/A = 0; the
            // coefficient (e^{dA}-1)/A -> delta there) or A > 0
#pragma unroll
            for (int k = 0; k < K; ++k) {
              const float z = dt[k] * a2;
              a[k] = fast_exp2(z);
              const float coef = ia == 0.0f ? dt[k] : expm1_zoh(z, a[k]) * ia;
              beta[k] = coef * Bv[k] * uv[k];
              if constexpr (RST) a[k] *= keep[k];
              agg = k == 0 ? beta[0] : __builtin_fmaf(a[k], agg, beta[k]);
            }
          }
          float Ag = fast_exp2(a2 * dsum);
          if constexpr (RST) Ag *= lane_keep;
          // the carried state enters through the first lane's summary
          agg = (j == 0) ? __builtin_fmaf(Ag, cr[n], agg) : agg;
          affine_scan_inclusive_fused<R>(Ag, agg);
          const float hend = agg;                        // state after this lane's steps
          if constexpr (!STATES) {
            float h = group_shift_right<R>(hend, cr[n]);  // state before them
#pragma unroll
            for (int k = 0; k < K; ++k) {
              h = __builtin_fmaf(a[k], h, beta[k]);
              y[k] = __builtin_fmaf(Cv[k], h, y[k]);
            }
          }
          cr[n] = last_to_first<R>(hend);                // state after the chunk
        }
        mem_fence_compiler();
      }

      if constexpr (!STATES) {
        if (z_row) {
#pragma unroll
          for (int k = 0; k < K; ++k) y[k] *= silu(zv[k]);
        }
        if (active)
          store_items<T, K>(OPQ ? static_cast<T*>(p.out) + lane_row() : out_row, tl, L, full, y);
      }
      if (more) store_state(ch + 1);
      if constexpr (TILE) {
        if (more) stage.store(reinterpret_cast<float*>(tile_mem[buf ^ 1]), N, tid_o());
        __syncthreads();
      }
    }
  };
  if (ZOH && any_tiny) run_chunks(std::true_type{});
  else run_chunks(std::false_type{});

  // one pass: the last state (segmented runs: the carry kernel writes it)
  if (MODE == kModeOut && SEG == kSegWhole && p.nseg == 1 && active && j == 0 && p.last_state) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (n < N) p.last_state[c * N + n] = cr[n];
  }
  if constexpr (LOCAL || MODE == kModeSegSummary) {
    const float dseg = group_sum<R>(dtot);
    const float nreset = group_sum<R>(seg_reset ? 1.0f : 0.0f);
    if (active && j == 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
        if (n < N) p.seg_state[(c * p.nseg + seg) * N + n] = cr[n];
      p.seg_dsum[c * p.nseg + seg] = dseg;
      p.seg_keep[c * p.nseg + seg] = nreset > 0.0f ? 0.0f : 1.0f;
    }
  }
}

template <typename T, int R, int K, int NT, bool ZOH, bool VEC, int MODE, bool RST = false,
          bool EXACT = false, int SEG = kSegWhole>
static hipError_t launch_fwd(const FwdParams& p, hipStream_t s) {
  const int64_t nblocks = p.batch * p.groups * p.nseg;
  hipLaunchKernelGGL((scan_fwd_kernel<T, R, K, NT, ZOH, VEC, MODE, RST, EXACT, SEG>),
                     dim3((unsigned)nblocks), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

// N <= 16 takes the NT = 16 kernel, 16 < N <= 64 the NT = 64 kernel; with
// 16 lanes per channel, N == 16 (the usual state size) has a variant of its own.
template <typename T, int R, int K, bool ZOH, int MODE, bool RST = false, int SEG = kSegWhole>
static hipError_t fwd_nv(const FwdParams& p, bool vec, hipStream_t s) {
  if constexpr (R == 16) {
    if (p.N == 16)
      return vec ? launch_fwd<T, R, K, 16, ZOH, true, MODE, RST, true, SEG>(p, s)
                 : launch_fwd<T, R, K, 16, ZOH, false, MODE, RST, true, SEG>(p, s);
  }
  if (p.N <= 16)
    return vec ? launch_fwd<T, R, K, 16, ZOH, true, MODE, RST, false, SEG>(p, s)
               : launch_fwd<T, R, K, 16, ZOH, false, MODE, RST, false, SEG>(p, s);
  return vec ? launch_fwd<T, R, K, 64, ZOH, true, MODE, RST, false, SEG>(p, s)
             : launch_fwd<T, R, K, 64, ZOH, false, MODE, RST, false, SEG>(p, s);
}

// 16 lanes per channel, the segment pass from p.seg_pass (first launch) or
// kSegFix (second launch of a segmented run).
template <typename T, int K, bool ZOH, int MODE, bool RST, bool FIX>
static hipError_t fwd_seg16(const FwdParams& p, bool vec, hipStream_t s) {
  if constexpr (FIX) {
    return fwd_nv<T, 16, K, ZOH, MODE, RST, kSegFix>(p, vec, s);
  } else {
    if (p.seg_pass == kSegLocal) return fwd_nv<T, 16, K, ZOH, MODE, RST, kSegLocal>(p, vec, s);
    return fwd_nv<T, 16, K, ZOH, MODE, RST, kSegWhole>(p, vec, s);
  }
}

// Reset flags: 16 lanes per channel only.
template <typename T, int K, int MODE, bool FIX = false>
static hipError_t dispatch_fwd_reset_t(const FwdParams& p, int disc, bool vec, hipStream_t s) {
  return disc == 0 ? fwd_seg16<T, K, true, MODE, true, FIX>(p, vec, s)
                   : fwd_seg16<T, K, false, MODE, true, FIX>(p, vec, s);
}

// The second launch of a segmented run (no reset flags).
template <typename T, int K, int MODE>
static hipError_t dispatch_fwd_fix_t(const FwdParams& p, int disc, bool vec, hipStream_t s) {
  return disc == 0 ? fwd_seg16<T, K, true, MODE, false, true>(p, vec, s)
                   : fwd_seg16<T, K, false, MODE, false, true>(p, vec, s);
}

template <typename T, int K, int MODE>
static hipError_t dispatch_fwd_t(const FwdParams& p, int disc, int lanes, bool vec,
                                 hipStream_t s) {
  const bool zoh = disc == 0;
  switch (lanes) {
    case 16:
      return zoh ? fwd_seg16<T, K, true, MODE, false, false>(p, vec, s)
                 : fwd_seg16<T, K, false, MODE, false, false>(p, vec, s);
    case 32:
      return zoh ? fwd_nv<T, 32, K, true, MODE>(p, vec, s) : fwd_nv<T, 32, K, false, MODE>(p, vec, s);
    default:
      return zoh ? fwd_nv<T, 64, K, true, MODE>(p, vec, s) : fwd_nv<T, 64, K, false, MODE>(p, vec, s);
  }
}

}  // namespace mscan

// Complex-valued selective scan, forward: diagonal complex A, complex B, C
// and state (the S4D-Lin parameterization A_n = -1/2 + i*pi*n that the
// paper-graph-ui summary, section 3.4 "Real vs. Complex", and the
// trishampatil essay, Part III, describe for audio).  Per channel (b, d):
//   Abar = exp(delta A),  Bbar = (Abar - 1)/A B (ZOH; delta B at A = 0) or delta B
//   h_t = Abar h_{t-1} + Bbar u_t,  y_t = Re(sum_n C_t[n] h_t[n]) + D u_t
//   out = y * SiLU(z)
// (the output convention is the plain reading: the pages fix none).
//
// Layout and decomposition follow the real forward: 16 lanes per channel
// along time, 8 steps per lane (128-step chunks), 4 channels per wave and 16
// per block of one batch row.  The affine pairs (Abar, Bbar u) are complex;
// the 16-lane scan combines them with DPP row shifts (row_shr 1, 2, 4, 8; a
// lane without a source takes the identity pair).  The carry per (channel,
// state) lives in LDS and enters through lane 0.  Complex arrays are
// interleaved (re, im) float pairs.
#include "device_common.hpp"
#include "kernels.hpp"
#include "complex_common.hpp"
#include "scan_fwd_impl.hpp"
#include "tile_stage.hpp"

namespace mscan {

namespace {

constexpr int R = 16;
constexpr int K = 8;
constexpr int CPB = (kBlock / 64) * (64 / R);
constexpr int TCH = R * K;
constexpr int NT = 16;

// MODE 0: the outputs, and the chunk states too when p.chunk_states is set
// (checkpoints for a later backward).  MODE 1: the backward's recompute pass,
// only the state entering every chunk (to p.chunk_states).  MODE 2: the
// summary pass of a segmented run, each segment's end state from a zero start
// and its decay prod(Abar) per state (p.seg_state, p.seg_dec).  Modes 1 and 2
// skip C, y and out.
//
// A block serves one channel group of one batch row for the whole sequence
// or, in a segmented run (p.seg_chunks > 0), for one segment of it; the
// output and state passes then start each segment from p.seg_h0, which the
// carry kernel below filled from the summaries (the associative combination
// of trishampatil essay, Part III §2, on whole segments).
//
// RST: packed sequences.  Where p.reset flags a step the state entering it
// is zero: the step's decay in the recurrence (not in Bbar) becomes 0, and so
// does the decay of any lane summary that holds the step (the segment's
// product of Abar then vanishes too, so the carry passes nothing across it).
//
// B and C (complex, shared by the block's 16 channels) are staged per chunk
// into one LDS tile by the whole block with 16-byte loads (tile_stage.hpp:
// a complex row of TCH steps is a float row of 2*TCH); the next chunk's
// loads are in flight in registers while the current chunk computes.
template <typename T, bool ZOH, bool VEC, int MODE, bool RST>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void scan_fwd_complex_kernel(
    const CplxParams p) {
  constexpr bool STATES = MODE != 0;
  constexpr bool SUMMARY = MODE == 2;
  constexpr int ROWS = STATES ? NT : 2 * NT;   // B rows, then C rows
  constexpr int RW = 2 * TCH;                  // floats per tile row
  __shared__ float4 tile_mem[ROWS * RW / 4];
  // {A.re log2(e), A.im / (2 pi), (1/A).re, (1/A).im}; 1/A = 0 where A ~ 0
  __shared__ float4 prm[CPB][NT];
  __shared__ float2 carry[CPB][NT];
  __shared__ float2 decs[SUMMARY ? CPB : 1][NT];   // summary: prod(Abar) so far

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane % R;
  const int cl = (tid >> 6) * (64 / R) + lane / R;
  // block order (b, segment, group) with the group fastest
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_b = p.groups * p.nseg;
  const int64_t b = blk / per_b;
  const int64_t seg = (blk - b * per_b) / p.groups;
  const int64_t grp = blk - b * per_b - seg * p.groups;
  const int64_t d_raw = grp * CPB + cl;
  const bool active = d_raw < p.dim;
  const int64_t d = active ? d_raw : p.dim - 1;
  const int64_t c = b * p.dim + d;
  const int N = p.N;
  const int64_t L = p.L;

  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    const bool real = dd < p.dim && n < N;
    const float2 a = real ? p.A[dd * N + n] : make_float2(-1.0f, 0.0f);
    const float m2 = a.x * a.x + a.y * a.y;
    const bool tiny = __builtin_fabsf(a.x) < 1e-30f && __builtin_fabsf(a.y) < 1e-30f;
    const float2 ia = tiny ? make_float2(0.0f, 0.0f) : make_float2(a.x / m2, -a.y / m2);
    prm[ci][n] = make_float4(a.x * kLog2e, a.y * kInv2Pi, ia.x, ia.y);
    const int64_t cc = b * p.dim + dd;
    float2 h = make_float2(0.0f, 0.0f);
    if (real && !SUMMARY) {
      if (p.seg_h0) h = p.seg_h0[(cc * p.nseg + seg) * N + n];
      else if (p.h0) h = p.h0[cc * N + n];
    }
    carry[ci][n] = h;
    if constexpr (SUMMARY) decs[ci][n] = make_float2(1.0f, 0.0f);
  }

  const T* __restrict__ u_row = static_cast<const T*>(p.u) + c * L;
  const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + c * L;
  const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + c * L : nullptr;
  const float* __restrict__ Bf = reinterpret_cast<const float*>(p.B) + b * N * 2 * L;
  const float* __restrict__ Cf = reinterpret_cast<const float*>(p.C) + b * N * 2 * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const uint8_t* __restrict__ rst_row = RST ? p.reset + b * L : nullptr;
  const int64_t nchunks = (L + TCH - 1) / TCH;
  const int64_t ch_begin = p.seg_chunks > 0 ? seg * p.seg_chunks : 0;
  const int64_t ch_end =
      p.seg_chunks > 0 ? (ch_begin + p.seg_chunks < nchunks ? ch_begin + p.seg_chunks : nchunks)
                       : nchunks;
  float* tile = reinterpret_cast<float*>(tile_mem);

  TileStager<float, RW, 2 * K, NT, ROWS, kBlock> stage;
  stage.load(Bf, Cf, N, 2 * L, 2 * ch_begin * TCH, VEC && (ch_begin + 1) * TCH <= L, tid);
  stage.store(tile, N, tid);
  __syncthreads();

  for (int64_t ch = ch_begin; ch < ch_end; ++ch) {
    const int64_t tl = ch * TCH + (int64_t)j * K;
    const bool full = VEC && ch * TCH + TCH <= L;
    const bool more = ch + 1 < ch_end;
    if (more) stage.load(Bf, Cf, N, 2 * L, 2 * (ch + 1) * TCH, VEC && (ch + 2) * TCH <= L, tid);
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    // the state entering the chunk: the backward's recompute pass, or the
    // checkpoints a forward may save for a later backward
    if (!SUMMARY && (STATES || p.chunk_states) && active && j == 0) {
      for (int n = 0; n < N; ++n) p.chunk_states[(c * nchunks + ch) * N + n] = carry[cl][n];
    }
    float uv[K], dt[K], y[K];
    load_items<T, K>(u_row, tl, L, full, uv);
    load_items<T, K>(dl_row, tl, L, full, dt);
    float dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float r = dt[k] + bias;
      const float s = p.softplus ? softplus(r) : r;
      dt[k] = k < nvalid ? s : 0.0f;       // steps past L are the identity map
      dsum += dt[k];
      y[k] = Dd * uv[k];
    }
    float keep[K];
    float lane_keep = 1.0f;
    if constexpr (RST) lane_keep = load_keep<K>(rst_row, tl, L, keep) ? 0.0f : 1.0f;

    for (int n = 0; n < N; ++n) {
      const float4 pr = prm[cl][n];
      const float ar2 = pr.x, air = pr.y;
      const float2 ia = make_float2(pr.z, pr.w);
      const bool tiny = ZOH && ia.x == 0.0f && ia.y == 0.0f;
      float bf[2 * K];
      tile_read<2 * K>(tile + n * RW, j, bf);   // steps past L were staged as 0
      float2 ab[K], beta[K];
      if (!ZOH || __builtin_amdgcn_ballot_w64(tiny) == 0) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float2 Bu = make_float2(bf[2 * k] * uv[k], bf[2 * k + 1] * uv[k]);
          if constexpr (ZOH) {
            float2 em1;
            ab[k] = cexp_expm1_scaled(dt[k], ar2, air, em1);
            beta[k] = cmul(em1, cmul(ia, Bu));      // (Abar - 1)/A B u
          } else {
            ab[k] = cexp_scaled(dt[k], ar2, air);
            beta[k] = cscale(Bu, dt[k]);
          }
        }
      } else {
        // a channel of this wave has A ~ 0 (1/A stored as 0): delta B u there
#pragma unroll
        for (int k = 0; k < K; ++k) {
          float2 em1;
          ab[k] = cexp_expm1_scaled(dt[k], ar2, air, em1);
          const float2 Bu = make_float2(bf[2 * k] * uv[k], bf[2 * k + 1] * uv[k]);
          beta[k] = tiny ? cscale(Bu, dt[k]) : cmul(em1, cmul(ia, Bu));
        }
      }
      if constexpr (RST) {
#pragma unroll
        for (int k = 0; k < K; ++k) ab[k] = cscale(ab[k], keep[k]);   // the decay only
      }
      float2 agg = beta[0];
#pragma unroll
      for (int k = 1; k < K; ++k) agg = cfma(ab[k], agg, beta[k]);
      // the lane's decay: exp(A * sum of its steps)
      float2 Ag = cexp_scaled(dsum, ar2, air);
      if constexpr (RST) Ag = cscale(Ag, lane_keep);
      const float2 cin = carry[cl][n];
      if (j == 0) agg = cfma(Ag, cin, agg);    // the carried state enters lane 0
      cplx_scan_prefix_row(Ag, agg);
      if constexpr (!STATES) {
        float cf[2 * K];
        tile_read<2 * K>(tile + (NT + n) * RW, j, cf);
        // state before this lane's steps: the previous lane's end (lane 0: the carry)
        float2 h = make_float2(dpp_mov<kRowShr1>(cin.x, agg.x), dpp_mov<kRowShr1>(cin.y, agg.y));
#pragma unroll
        for (int k = 0; k < K; ++k) {
          h = cfma(ab[k], h, beta[k]);
          y[k] = __builtin_fmaf(cf[2 * k], h.x, __builtin_fmaf(-cf[2 * k + 1], h.y, y[k]));
        }
      }
      // all lanes have read carry[cl][n] above; lane 15 holds the chunk's end
      // (and, after the scan, the chunk's decay prod(Abar) in Ag)
      if (j == R - 1) {
        carry[cl][n] = agg;
        if constexpr (SUMMARY) decs[cl][n] = cmul(Ag, decs[cl][n]);
      }
    }

    if constexpr (!STATES) {
      if (z_row) {
        float zv[K];
        load_items<T, K>(z_row, tl, L, full, zv);
#pragma unroll
        for (int k = 0; k < K; ++k) y[k] *= silu(zv[k]);
      }
      if (active) store_items<T, K>(static_cast<T*>(p.out) + c * L, tl, L, full, y);
    }
    // every wave is done with this chunk's tile: write the next one
    __syncthreads();
    if (more) {
      stage.store(tile, N, tid);
      __syncthreads();
    }
  }

  // one pass: the last state (segmented runs: the carry kernel writes it)
  if (!STATES && p.nseg == 1 && p.last_state && active && j == 0) {
    for (int n = 0; n < N; ++n) p.last_state[c * N + n] = carry[cl][n];
  }
  if constexpr (SUMMARY) {
    // the loop's last barrier has made every lane 15's writes visible
    if (active && j == 0) {
      const int64_t k = (c * p.nseg + seg) * N;
      for (int n = 0; n < N; ++n) {
        p.seg_state[k + n] = carry[cl][n];
        p.seg_dec[k + n] = decs[cl][n];
      }
    }
  }
}

// One thread per (channel, n): the state entering segment s + 1 is the one
// entering s times the segment's decay plus its end state from zero.
__global__ __launch_bounds__(256) void seg_carry_complex_kernel(const CplxParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.nchannels * p.N) return;
  const int64_t c = i / p.N;
  const int n = (int)(i - c * p.N);
  float2 H = p.h0 ? p.h0[c * p.N + n] : make_float2(0.0f, 0.0f);
  for (int64_t s = 0; s < p.nseg; ++s) {
    const int64_t k = (c * p.nseg + s) * p.N + n;
    p.seg_h0[k] = H;
    H = cfma(p.seg_dec[k], H, p.seg_state[k]);
  }
  if (p.last_state) p.last_state[c * p.N + n] = H;
}

template <typename T, int MODE, bool RST>
hipError_t launch_complex_rst(const CplxParams& p, int disc, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)(p.batch * p.groups * p.nseg)), block(kBlock);
  if (disc == 0) {
    if (vec) hipLaunchKernelGGL((scan_fwd_complex_kernel<T, true, true, MODE, RST>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((scan_fwd_complex_kernel<T, true, false, MODE, RST>), grid, block, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((scan_fwd_complex_kernel<T, false, true, MODE, RST>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((scan_fwd_complex_kernel<T, false, false, MODE, RST>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <typename T, int MODE>
hipError_t launch_complex(const CplxParams& p, int disc, bool vec, hipStream_t s) {
  return p.reset ? launch_complex_rst<T, MODE, true>(p, disc, vec, s)
                 : launch_complex_rst<T, MODE, false>(p, disc, vec, s);
}

}  // namespace

hipError_t dispatch_scan_fwd_complex(const CplxParams& p, int dtype, int disc, bool vec,
                                     hipStream_t s) {
  return dtype == 0 ? launch_complex<float, 0>(p, disc, vec, s)
                    : launch_complex<bf16_t, 0>(p, disc, vec, s);
}

hipError_t dispatch_chunk_states_complex(const CplxParams& p, int dtype, int disc, bool vec,
                                         hipStream_t s) {
  return dtype == 0 ? launch_complex<float, 1>(p, disc, vec, s)
                    : launch_complex<bf16_t, 1>(p, disc, vec, s);
}

hipError_t dispatch_seg_summary_complex(const CplxParams& p, int dtype, int disc, bool vec,
                                        hipStream_t s) {
  return dtype == 0 ? launch_complex<float, 2>(p, disc, vec, s)
                    : launch_complex<bf16_t, 2>(p, disc, vec, s);
}

hipError_t dispatch_seg_carry_complex(const CplxParams& p, hipStream_t s) {
  const int64_t blocks = (p.nchannels * p.N + 255) / 256;
  hipLaunchKernelGGL(seg_carry_complex_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mscan

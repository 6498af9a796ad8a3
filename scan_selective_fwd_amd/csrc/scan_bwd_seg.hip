// Segmented backward, adjoint side: the summary of each segment's adjoint and
// the carry over segments in reverse order.
//
// The adjoint of the reverse recurrence, g_t = Abar_t (g_{t+1} + C_t gy_t)
// (scan_bwd_impl.hpp), is an affine map per step of the same kind as the
// forward's (Abar, Bbar u) pairs, composed from the later step to the earlier
// one.  Over a whole segment it is  g_start = G + exp(A sum(delta)) g_end,
// with G the segment's adjoint at its first step when zero enters its end.
// The summary kernel computes G, the delta sum and a reset-free factor for
// every (channel, segment) in parallel; the carry kernel walks the segments of
// each (channel, state) from last to first to get the adjoint entering each
// segment from the right.  This is the associative combination the pages'
// parallel scan rests on (trishampatil essay, Part III §2), applied in reverse
// time to whole segments of the chunked scan of its Part III §4; the backward
// kernel then runs every segment from its entering adjoint.  A segment that
// contains a reset flag passes nothing on (its keep factor is 0): the adjoint
// of the state entering a flagged step is zero.
#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_fwd_impl.hpp"
#include "tile_stage.hpp"

namespace mscan {

// One block per (batch row, segment, channel group): 16 channels, 16 lanes
// each, 8 steps per lane, the chunks of the segment from last to first.  NT =
// 16 stages the C rows of a chunk in LDS (double buffered); NT = 64 reads them
// per lane from global memory.
template <typename T, int NT, bool VEC, bool RST>
__global__ __launch_bounds__(kBlock) void bwd_seg_summary_kernel(const BwdParams p) {
  constexpr int R = 16;
  constexpr int K = kItemsBwd;
  constexpr int CPW = 64 / R;
  constexpr int CPB = (kBlock / 64) * CPW;
  constexpr int TCH = R * K;
  constexpr bool TILE = (NT == 16);
  __shared__ float4 tile_mem[2][TILE ? NT * TCH / 4 : 1];
  __shared__ float a2s[CPB][NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane % R;
  const int cl = wave * CPW + lane / R;
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

  const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + c * L;
  const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + c * L : nullptr;
  const T* __restrict__ do_row = static_cast<const T*>(p.dout) + c * L;
  const T* __restrict__ C_b = static_cast<const T*>(p.C) + b * N * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const uint8_t* __restrict__ rst_row = RST ? p.reset + b * L : nullptr;

  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    a2s[ci][n] = (dd < p.dim && n < N) ? p.A[dd * N + n] * kLog2e : 0.0f;
  }

  const int64_t nchunks = p.nchunks;
  const int64_t ch_begin = seg * p.seg_chunks;
  const int64_t ch_end =
      ch_begin + p.seg_chunks < nchunks ? ch_begin + p.seg_chunks : nchunks;

  // only the C rows are staged (tile row n = C row n)
  TileStager<T, TCH, K, NT, TILE ? NT : 1, kBlock> stage;
  if constexpr (TILE) {
    const int64_t tb = (ch_end - 1) * TCH;
    stage.load(C_b, C_b, N, L, tb, VEC && tb + TCH <= L, tid);
    stage.store(reinterpret_cast<float*>(tile_mem[0]), N, tid);
  }
  __syncthreads();

  // adjoint entering the current chunk from the right, per state, in lane 15
  float gc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) gc[n] = 0.0f;
  float dtot = 0.0f;
  bool seg_reset = false;

  for (int64_t ch = ch_end - 1; ch >= ch_begin; --ch) {
    const int buf = (int)((ch_end - 1 - ch) & 1);
    const int64_t t0 = ch * TCH;
    const int64_t tl = t0 + (int64_t)j * K;
    const bool full = VEC && t0 + TCH <= L;
    const bool more = ch > ch_begin;
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    if constexpr (TILE) {
      if (more) stage.load(C_b, C_b, N, L, t0 - TCH, VEC, tid);   // earlier chunks are full
    }
    float dt[K], gy[K];
    {
      float raw[K];
      load_items<T, K>(dl_row, tl, L, full, raw);
      load_items<T, K>(do_row, tl, L, full, gy);
      if (z_row) {
        float zv[K];
        load_items<T, K>(z_row, tl, L, full, zv);
#pragma unroll
        for (int k = 0; k < K; ++k) gy[k] *= silu(zv[k]);
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float r = raw[k] + bias;
        const float s = p.softplus ? softplus(r) : r;
        dt[k] = (k < nvalid) ? s : 0.0f;   // steps past L are the identity map
        gy[k] = active ? gy[k] : 0.0f;
      }
    }
    float dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) dsum += dt[k];
    dtot += dsum;
    float keep[K];
    float lane_keep = 1.0f;
    if constexpr (RST) {
      const bool any = load_keep<K>(rst_row, tl, L, keep);
      lane_keep = any ? 0.0f : 1.0f;
      seg_reset |= any;
    }

    const float* tC = reinterpret_cast<const float*>(tile_mem[buf]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n < N) {
        const float a2 = a2s[cl][n];
        float Cv[K];
        if constexpr (TILE) tile_read<K>(tC + n * TCH, j, Cv);
        else load_items<T, K>(C_b + (int64_t)n * L, tl, L, full, Cv);
        // this lane's steps, later first: g <- Abar (g + C gy)
        float gagg = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
          float a = fast_exp2(dt[k] * a2);
          if constexpr (RST) a *= keep[k];
          gagg = a * __builtin_fmaf(Cv[k], gy[k], gagg);
        }
        float As = fast_exp2(a2 * dsum);
        if constexpr (RST) As *= lane_keep;
        gagg = (j == R - 1) ? __builtin_fmaf(As, gc[n], gagg) : gagg;   // later chunk enters lane 15
        affine_suffix_scan_row_fused(As, gagg);
        gc[n] = row_first_to_last(gagg);   // adjoint at the chunk start, to lane 15
      }
      mem_fence_compiler();
    }
    if constexpr (TILE) {
      if (more) stage.store(reinterpret_cast<float*>(tile_mem[buf ^ 1]), N, tid);
      __syncthreads();
    }
  }

  const float dseg = group_sum<R>(dtot);
  const float nreset = group_sum<R>(seg_reset ? 1.0f : 0.0f);
  if (active && j == R - 1) {
    const int64_t k = c * p.nseg + seg;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (n < N) p.seg_gloc[k * N + n] = gc[n];
    p.seg_gdsum[k] = dseg;
    p.seg_gkeep[k] = nreset > 0.0f ? 0.0f : 1.0f;
  }
}

// One thread per (channel, n): g entering segment s from the right is the
// adjoint at the start of segment s + 1, i.e. that segment's summary plus its
// decay times the adjoint entering it; zero enters the last segment.
static __global__ __launch_bounds__(256) void bwd_seg_carry_kernel(const BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.nchannels * p.N) return;
  const int64_t c = i / p.N;
  const int n = (int)(i - c * p.N);
  const int64_t d = c % p.dim;
  const float a2 = p.A[d * p.N + n] * kLog2e;
  float G = 0.0f;
  for (int64_t s = p.nseg - 1; s >= 0; --s) {
    const int64_t k = c * p.nseg + s;
    p.seg_gin[k * p.N + n] = G;
    const float decay = exp2f(a2 * p.seg_gdsum[k]) * p.seg_gkeep[k];
    G = __builtin_fmaf(decay, G, p.seg_gloc[k * p.N + n]);
  }
}

template <typename T, int NT, bool RST>
static hipError_t launch_bwd_seg_summary(const BwdParams& p, bool vec, hipStream_t s) {
  const int64_t nblocks = p.batch * p.groups * p.nseg;
  if (vec)
    hipLaunchKernelGGL((bwd_seg_summary_kernel<T, NT, true, RST>), dim3((unsigned)nblocks),
                       dim3(kBlock), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_seg_summary_kernel<T, NT, false, RST>), dim3((unsigned)nblocks),
                       dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

template <typename T, bool RST>
static hipError_t bwd_seg_summary_nt(const BwdParams& p, bool vec, hipStream_t s) {
  return p.N <= 16 ? launch_bwd_seg_summary<T, 16, RST>(p, vec, s)
                   : launch_bwd_seg_summary<T, 64, RST>(p, vec, s);
}

hipError_t dispatch_bwd_seg_summary(const BwdParams& p, int dtype, bool vec, hipStream_t s) {
  if (p.reset)
    return dtype == 0 ? bwd_seg_summary_nt<float, true>(p, vec, s)
                      : bwd_seg_summary_nt<bf16_t, true>(p, vec, s);
  return dtype == 0 ? bwd_seg_summary_nt<float, false>(p, vec, s)
                    : bwd_seg_summary_nt<bf16_t, false>(p, vec, s);
}

hipError_t dispatch_bwd_seg_carry(const BwdParams& p, hipStream_t s) {
  const int64_t total = p.nchannels * p.N;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(bwd_seg_carry_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mscan

// Complex-valued selective scan, backward (for scan_fwd_complex.hip): the
// states are recomputed chunkwise from the state entering each 128-step
// chunk (paper-graph-ui summary, section 3.4, and trishampatil essay, Part
// III §4: the expanded states are recomputed, not stored), the adjoint runs
// in reverse time as a complex affine scan, and every gradient is formed.
//
// With the gradient of a complex w written g_w = dL/dRe(w) + i dL/dIm(w) and
// gy_t = dout_t * SiLU(z_t), the chain rule of the forward gives
//   G_t = conj(C_t) gy_t + conj(Abar_{t+1}) G_{t+1}           (adjoint of h_t)
//   ddelta_t += Re(conj(G) Abar (A h_{t-1} + B u))            (ZOH; Euler: A Abar h + B u)
//   dA  += conj((delta Abar (A h_{t-1} + B u) - Bbar u) / A) G (ZOH; limits at A = 0)
//   du_t += Re(conj(G) E B),  dB_t += u conj(E) G,  dC_t += gy conj(h_t)
// where E = Bbar / B.  Structure as in the real backward: 16 channels of one
// batch row per block, 16 lanes per channel along time, 8 steps per lane;
// per chunk (last to first) and state index: replay (prefix scan), adjoint
// (suffix scan, the later chunk's adjoint entering lane 15), gradients.  dB
// and dC are summed over the wave's 4 channels with permlane swaps, over the
// block's waves through per-wave LDS slices, and into global memory with one
// float atomic per (n, t, re/im) per block.  B and C of a chunk are staged
// once per block into an LDS tile (tile_stage.hpp; a complex row of TCH steps
// is a float row of 2*TCH); the earlier chunk's loads are issued after the
// state loop and written to the tile at the chunk's end.
//
// Long sequences with few channels are split into segments of whole chunks,
// one block per (batch row, segment, channel group), as in the real backward:
// the adjoint entering a segment from the right comes from the segments after
// it, each of which maps the adjoint at its end to G + conj(prod Abar) times
// it, G being its adjoint at its start from a zero end.  The summary and
// carry kernels at the end of this file compute those; only segment 0 writes
// dh0.
//
// RST: packed sequences (p.reset flags), as in the real backward: a flagged
// step's decay becomes 0 in the recurrence and the adjoint (Bbar, and the
// Abar in its derivatives, keep the true value), its h_{t-1} counts as 0, and
// no adjoint passes back across it.
#include "complex_common.hpp"
#include "kernels.hpp"
#include "scan_fwd_impl.hpp"
#include "tile_stage.hpp"

namespace mscan {

namespace {

constexpr int R = 16;
constexpr int K = 8;
constexpr int CPB = (kBlock / 64) * (64 / R);
constexpr int TCH = R * K;
constexpr int NT = 16;
constexpr int G = 2;                 // state indices per dB/dC flush
constexpr int NW = kBlock / 64;

template <typename T, bool ZOH, bool VEC, bool RST>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void scan_bwd_complex_kernel(
    const CplxBwdParams p) {
  __shared__ float4 prm[CPB][NT];            // {A, 1/A} (1/A = 0 where A ~ 0)
  __shared__ float2 prs[CPB][NT];            // {A.re log2(e), A.im / (2 pi)}
  __shared__ float2 gcs[CPB][NT];            // adjoint entering from the later chunk
  __shared__ float2 dAs[CPB][NT];            // dA of each channel, this batch row
  __shared__ float red[2][NW][4][G][TCH];    // dB.re, dB.im, dC.re, dC.im partials per wave
  constexpr int RW = 2 * TCH;                // floats per tile row
  __shared__ float4 tile_mem[2 * NT * RW / 4];   // B rows, then C rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane % R;
  const int row = lane / R;
  const int cl = wave * (64 / R) + row;
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
  const int64_t nchunks = p.nchunks;
  const int64_t ch_begin = p.seg_chunks > 0 ? seg * p.seg_chunks : 0;
  const int64_t ch_end =
      p.seg_chunks > 0 ? (ch_begin + p.seg_chunks < nchunks ? ch_begin + p.seg_chunks : nchunks)
                       : nchunks;

  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    const bool real = dd < p.dim && n < N;
    const float2 a = real ? p.A[dd * N + n] : make_float2(-1.0f, 0.0f);
    const float m2 = a.x * a.x + a.y * a.y;
    const bool tiny = __builtin_fabsf(a.x) < 1e-30f && __builtin_fabsf(a.y) < 1e-30f;
    const float2 ia = tiny ? make_float2(0.0f, 0.0f) : make_float2(a.x / m2, -a.y / m2);
    prm[ci][n] = make_float4(a.x, a.y, ia.x, ia.y);
    prs[ci][n] = make_float2(a.x * kLog2e, a.y * kInv2Pi);
    // the adjoint entering the block's last chunk: zero at the sequence end
    // (no gradient flows into the final state), else the later segments'
    gcs[ci][n] = (real && p.seg_gin) ? p.seg_gin[((b * p.dim + dd) * p.nseg + seg) * N + n]
                                     : make_float2(0.0f, 0.0f);
    dAs[ci][n] = make_float2(0.0f, 0.0f);
  }
  __syncthreads();

  // the channel row as block-uniform base + lane part; row addresses are
  // formed from an opaque copy of the lane part where they are used, so that
  // none is kept (and spilled) across the chunk loop
  const int64_t c_blk = b * p.dim + grp * CPB;
  const int cl_eff = (int)(d - grp * CPB);
  auto row_off = [&]() { return (c_blk + opaque_int(cl_eff)) * L; };
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const uint8_t* __restrict__ rst_row = RST ? p.reset + b * L : nullptr;
  float dD_acc = 0.0f, db_acc = 0.0f;
  const float* __restrict__ Bf = reinterpret_cast<const float*>(p.B) + b * N * 2 * L;
  const float* __restrict__ Cf = reinterpret_cast<const float*>(p.C) + b * N * 2 * L;
  float* tile = reinterpret_cast<float*>(tile_mem);
  TileStager<float, RW, 2 * K, NT, 2 * NT, kBlock> stage;
  stage.load(Bf, Cf, N, 2 * L, 2 * (ch_end - 1) * TCH, VEC && ch_end * TCH <= L,
             opaque_int(tid));
  stage.store(tile, N, opaque_int(tid));
  __syncthreads();

  for (int64_t ch = ch_end - 1; ch >= ch_begin; --ch) {
    const int64_t t0 = ch * TCH;
    const int64_t tl = t0 + (int64_t)j * K;
    const bool full = VEC && t0 + TCH <= L;
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    float uv[K], dt[K], gy[K], yv[K], du[K], gdt[K];
    {
      const int64_t co = row_off();
      float raw[K], dov[K];
      load_items<T, K>(static_cast<const T*>(p.u) + co, tl, L, full, uv);
      load_items<T, K>(static_cast<const T*>(p.delta) + co, tl, L, full, raw);
      load_items<T, K>(static_cast<const T*>(p.dout) + co, tl, L, full, dov);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float r = raw[k] + bias;
        const float s = p.softplus ? softplus(r) : r;
        dt[k] = (k < nvalid) ? s : 0.0f;
        gy[k] = dov[k];
      }
      if (p.z) {
        float zv[K];
        load_items<T, K>(static_cast<const T*>(p.z) + co, tl, L, full, zv);
#pragma unroll
        for (int k = 0; k < K; ++k) gy[k] *= silu(zv[k]);
      }
    }
    float dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
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
    // a step's decay in the recurrence and the adjoint (0 at a flagged step)
    auto decay = [&](int k, float2 ab) { return RST ? cscale(ab, keep[k]) : ab; };

#pragma unroll 1
    for (int n = 0; n < N; ++n) {
      const float4 pr = prm[cl][n];
      const float2 a = make_float2(pr.x, pr.y), ia = make_float2(pr.z, pr.w);
      const float2 ps = prs[cl][n];
      const bool tiny = ZOH && ia.x == 0.0f && ia.y == 0.0f;
      const float2 h_in = p.chunk_states[(c * nchunks + ch) * N + n];
      const float2 gc = gcs[cl][n];
      // coef[k] = (Abar - 1)/A (its limit dt at A = 0; dt under Euler);
      // Bbar u = coef B u is formed where it is used
      float2 Bv[K], Cv[K], ab[K], coef[K], hv[K];
      auto read_bc = [&]() {
        float bf[2 * K], cf[2 * K];   // steps past L were staged as 0
        tile_read<2 * K>(tile + n * RW, j, bf);
        tile_read<2 * K>(tile + (NT + n) * RW, j, cf);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          Bv[k] = make_float2(bf[2 * k], bf[2 * k + 1]);
          Cv[k] = make_float2(cf[2 * k], cf[2 * k + 1]);
        }
      };
      read_bc();

      // ---- forward replay ----
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if constexpr (ZOH) {
          float2 em1;
          ab[k] = cexp_expm1_scaled(dt[k], ps.x, ps.y, em1);
          coef[k] = tiny ? make_float2(dt[k], 0.0f) : cmul(em1, ia);
        } else {
          ab[k] = cexp_scaled(dt[k], ps.x, ps.y);
          coef[k] = make_float2(dt[k], 0.0f);
        }
      }
      auto bbar_u = [&](int k) { return cmul(coef[k], cscale(Bv[k], uv[k])); };
      float2 agg = bbar_u(0);
#pragma unroll
      for (int k = 1; k < K; ++k) agg = cfma(decay(k, ab[k]), agg, bbar_u(k));
      const float2 Alane = RST ? cscale(cexp_scaled(dsum, ps.x, ps.y), lane_keep)
                               : cexp_scaled(dsum, ps.x, ps.y);
      float2 Ag = Alane;
      if (j == 0) agg = cfma(Ag, h_in, agg);
      cplx_scan_prefix_row(Ag, agg);
      const float2 hstart =
          make_float2(dpp_mov<kRowShr1>(h_in.x, agg.x), dpp_mov<kRowShr1>(h_in.y, agg.y));
      {
        float2 h = hstart;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          h = cfma(decay(k, ab[k]), h, bbar_u(k));
          hv[k] = h;
          yv[k] = __builtin_fmaf(Cv[k].x, h.x, __builtin_fmaf(-Cv[k].y, h.y, yv[k]));
        }
      }

      // ---- reverse adjoint: g leaving step t = conj(Abar_t) (conj(C_t) gy_t + g) ----
      float2 gagg = make_float2(0.0f, 0.0f);
#pragma unroll
      for (int k = K - 1; k >= 0; --k)
        gagg = cmul(cconj(decay(k, ab[k])), cadd(cscale(cconj(Cv[k]), gy[k]), gagg));
      float2 As = cconj(Alane);
      if (j == R - 1) gagg = cfma(As, gc, gagg);      // the later chunk enters lane 15
      cplx_scan_suffix_row(As, gagg);
      // adjoint arriving at each lane from the right (lane 15: the later chunk's)
      float2 g = make_float2(dpp_mov<0x101>(gc.x, gagg.x), dpp_mov<0x101>(gc.y, gagg.y));
      if (j == 0) gcs[cl][n] = gagg;                   // leaves the chunk at lane 0

      // B and C again from the tile (LDS): kept from the first reads, their
      // registers would be live across the scans (the fence keeps the
      // compiler from reusing those reads)
      mem_fence_compiler();
      read_bc();
      // ---- gradient terms ----
      // dA collects conj(dt Abar h_{t-1} + dcoef/dA B u) G: the Abar path and
      // (ZOH) the Bbar path, whose coefficient is formed without cancellation
      float2 dAc = make_float2(0.0f, 0.0f);
      float pv[4], sv[4][4], Tq[4][2];
#pragma unroll
      for (int k = K - 1; k >= 0; --k) {
        const float2 Gk = make_float2(__builtin_fmaf(Cv[k].x, gy[k], g.x),
                                      __builtin_fmaf(-Cv[k].y, gy[k], g.y));
        const float2 gn = cmul(cconj(ab[k]), Gk);   // with the true Abar
        float2 hprev = (k == 0) ? hstart : hv[k - 1];
        if constexpr (RST) hprev = cscale(hprev, keep[k]);
        const float2 Bu = cscale(Bv[k], uv[k]);
        const float2 Ah = cmul(ab[k], hprev);        // Abar h_{t-1}
        if constexpr (ZOH) {
          // ddelta: Re(conj(G) Abar (A h_{t-1} + B u)), dBbar/ddelta = Abar B
          const float2 W = cfma(a, Ah, cmul(ab[k], Bu));
          gdt[k] = __builtin_fmaf(Gk.x, W.x, __builtin_fmaf(Gk.y, W.y, gdt[k]));
          const float2 zeta = cdcoef_dA(dt[k], a, ab[k], coef[k], ia);
          dAc = cfma(cconj(cfma(zeta, Bu, cscale(Ah, dt[k]))), Gk, dAc);
        } else {
          gdt[k] += cdot(Gk, cmul(a, Ah)) + cdot(Gk, Bu);   // Euler: Bbar = dt B
          dAc = cfma(cconj(cscale(Ah, dt[k])), Gk, dAc);
        }
        // s = conj(E) G with E = Bbar / B; du and dB both use it
        const float2 sG = cmul(cconj(coef[k]), Gk);
        // Re(conj(G) E B) = Re(conj(s) B)
        du[k] = __builtin_fmaf(sG.x, Bv[k].x, __builtin_fmaf(sG.y, Bv[k].y, du[k]));
        const float2 vB = cscale(sG, uv[k]);
        const float2 vC = cscale(cconj(hv[k]), gy[k]);
        const float v[4] = {vB.x, vB.y, vC.x, vC.y};
        // sum over the wave's 4 channels, two steps at a time
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          if (k & 1) {
            pv[qq] = v[qq];
          } else {
            sv[qq][k / 2] = rs_pair16(v[qq], pv[qq]);
            if (k == 4) Tq[qq][1] = rs_pair32(sv[qq][2], sv[qq][3]);
            else if (k == 0) Tq[qq][0] = rs_pair32(sv[qq][0], sv[qq][1]);
          }
        }
        g = RST ? cscale(gn, keep[k]) : gn;   // the adjoint passed to step t - 1
      }
      const int buf = (n / G) & 1;
#pragma unroll
      for (int m = 0; m < 2; ++m) {   // lane (row r, j) owns step j*K + 4m + r
        const int pos = (4 * m + row) * 16 + j;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) red[buf][wave][qq][n % G][pos] = Tq[qq][m];
      }
      const float2 dAn = dAc;
      const float sx = row_sum_to_last(dAn.x);
      const float sy = row_sum_to_last(dAn.y);
      if (j == R - 1) dAs[cl][n] = cadd(dAs[cl][n], make_float2(sx, sy));

      if (n % G == G - 1 || n == N - 1) {
        // sum the waves' partials of this group of states into dB, dC
        // (block-uniform: N is the same for every thread)
        __syncthreads();
        const int n0 = n - (n % G);
        for (int s = 0; s < 4 * G * TCH / kBlock; ++s) {
          const int i = s * kBlock + tid;
          const int qq = i / (G * TCH);
          const int nn = (i / TCH) % G;
          const int tt = i % TCH;
          const int pos = (tt % K) * 16 + tt / K;
          float v = 0.0f;
#pragma unroll
          for (int w = 0; w < NW; ++w) v += red[buf][w][qq][nn][pos];
          if (n0 + nn < N && t0 + tt < L) {
            float* dst = reinterpret_cast<float*>(qq < 2 ? p.dB : p.dC);
            unsafeAtomicAdd(dst + 2 * ((b * N + n0 + nn) * L + t0 + tt) + (qq & 1), v);
          }
        }
      }
    }

    // the earlier chunk's B/C rows (every earlier chunk is whole)
    if (ch > ch_begin) stage.load(Bf, Cf, N, 2 * L, 2 * (ch - 1) * TCH, VEC, opaque_int(tid));

    // ---- per-step outputs ----
    const int64_t co = row_off();
    {
      float raw[K], ddl[K];
      load_items<T, K>(static_cast<const T*>(p.delta) + co, tl, L, full, raw);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float sg = p.softplus ? sigmoid(raw[k] + bias) : 1.0f;
        ddl[k] = (k < nvalid) ? gdt[k] * sg : 0.0f;
        db_acc += ddl[k];
      }
      if (active) {
        store_items<float, K>(p.du + co, tl, L, full, du);
        store_items<float, K>(p.ddelta + co, tl, L, full, ddl);
      }
    }
    if (p.z) {
      float zv[K], dov[K], dzv[K];
      load_items<T, K>(static_cast<const T*>(p.z) + co, tl, L, full, zv);
      load_items<T, K>(static_cast<const T*>(p.dout) + co, tl, L, full, dov);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float sg = sigmoid(zv[k]);
        dzv[k] = dov[k] * yv[k] * sg * __builtin_fmaf(zv[k], 1.0f - sg, 1.0f);
      }
      if (active) store_items<float, K>(p.dz + co, tl, L, full, dzv);
    }
    // keeps the next chunk's slice stores behind this chunk's flushes, and
    // every wave's tile reads behind the refill
    __syncthreads();
    if (ch > ch_begin) {
      stage.store(tile, N, opaque_int(tid));
      __syncthreads();
    }
  }

  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    if (dd < p.dim && n < N) {
      if (p.dh0 && seg == 0) p.dh0[(b * p.dim + dd) * N + n] = gcs[ci][n];
      float* dA = reinterpret_cast<float*>(p.dA + dd * N + n);
      unsafeAtomicAdd(dA, dAs[ci][n].x);
      unsafeAtomicAdd(dA + 1, dAs[ci][n].y);
    }
  }
  const float sD = row_sum_to_last(dD_acc);
  const float sb = row_sum_to_last(db_acc);
  if (active && j == R - 1) {
    if (p.dD) unsafeAtomicAdd(p.dD + d, sD);
    if (p.dbias) unsafeAtomicAdd(p.dbias + d, sb);
  }
}

__global__ __launch_bounds__(256) void cplx_bwd_zero_kernel(const CplxBwdParams p) {
  const int64_t nbc = 2 * p.batch * p.N * p.L;   // floats of dB (and of dC)
  const int64_t na = 2 * p.dim * p.N;
  const int64_t total = 2 * nbc + na + 2 * p.dim;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    if (i < nbc) reinterpret_cast<float*>(p.dB)[i] = 0.0f;
    else if (i < 2 * nbc) reinterpret_cast<float*>(p.dC)[i - nbc] = 0.0f;
    else if (i < 2 * nbc + na) reinterpret_cast<float*>(p.dA)[i - 2 * nbc] = 0.0f;
    else {
      const int64_t k = i - 2 * nbc - na;
      float* dst = k < p.dim ? p.dD : p.dbias;
      if (dst) dst[k < p.dim ? k : k - p.dim] = 0.0f;
    }
  }
}

// Adjoint summary of a segmented run: per (batch row, segment, group), the
// segment's chunks from last to first with a zero adjoint entering its end;
// per state, G (the adjoint at the segment's first step) and prod(conj Abar)
// over the segment.  Only delta, dout, z and C are read.
template <typename T, bool VEC, bool RST>
__global__ __launch_bounds__(kBlock) void bwd_seg_summary_complex_kernel(const CplxBwdParams p) {
  constexpr int RW = 2 * TCH;
  __shared__ float4 tile_mem[NT * RW / 4];   // C rows
  __shared__ float2 prs[CPB][NT];
  __shared__ float2 gcs[CPB][NT];            // adjoint entering the chunk from the right
  __shared__ float2 gds[CPB][NT];            // prod(conj Abar) over the chunks done

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane % R;
  const int cl = (tid >> 6) * (64 / R) + lane / R;
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
  const int64_t nchunks = p.nchunks;
  const int64_t ch_begin = seg * p.seg_chunks;
  const int64_t ch_end = ch_begin + p.seg_chunks < nchunks ? ch_begin + p.seg_chunks : nchunks;

  for (int i = tid; i < CPB * NT; i += kBlock) {
    const int ci = i / NT, n = i - ci * NT;
    const int64_t dd = grp * CPB + ci;
    const float2 a = (dd < p.dim && n < N) ? p.A[dd * N + n] : make_float2(-1.0f, 0.0f);
    prs[ci][n] = make_float2(a.x * kLog2e, a.y * kInv2Pi);
    gcs[ci][n] = make_float2(0.0f, 0.0f);
    gds[ci][n] = make_float2(1.0f, 0.0f);
  }

  const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + c * L;
  const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + c * L : nullptr;
  const T* __restrict__ do_row = static_cast<const T*>(p.dout) + c * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const uint8_t* __restrict__ rst_row = RST ? p.reset + b * L : nullptr;
  const float* __restrict__ Cf = reinterpret_cast<const float*>(p.C) + b * N * 2 * L;
  float* tile = reinterpret_cast<float*>(tile_mem);
  TileStager<float, RW, 2 * K, NT, NT, kBlock> stage;
  stage.load(Cf, Cf, N, 2 * L, 2 * (ch_end - 1) * TCH, VEC && ch_end * TCH <= L, tid);
  stage.store(tile, N, tid);
  __syncthreads();

  for (int64_t ch = ch_end - 1; ch >= ch_begin; --ch) {
    const int64_t tl = ch * TCH + (int64_t)j * K;
    const bool full = VEC && ch * TCH + TCH <= L;
    const int64_t rem = L - tl;
    const int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
    if (ch > ch_begin) stage.load(Cf, Cf, N, 2 * L, 2 * (ch - 1) * TCH, VEC, tid);
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
        const float sp = p.softplus ? softplus(r) : r;
        dt[k] = (k < nvalid) ? sp : 0.0f;   // steps past L are the identity map
        gy[k] = active ? gy[k] : 0.0f;
      }
    }
    float dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) dsum += dt[k];
    float keep[K];
    float lane_keep = 1.0f;
    if constexpr (RST) lane_keep = load_keep<K>(rst_row, tl, L, keep) ? 0.0f : 1.0f;

    for (int n = 0; n < N; ++n) {
      const float2 ps = prs[cl][n];
      float cf[2 * K];
      tile_read<2 * K>(tile + n * RW, j, cf);
      // this lane's steps, later first: g <- conj(Abar) (conj(C) gy + g)
      float2 gagg = make_float2(0.0f, 0.0f);
#pragma unroll
      for (int k = K - 1; k >= 0; --k) {
        float2 ab = cexp_scaled(dt[k], ps.x, ps.y);
        if constexpr (RST) ab = cscale(ab, keep[k]);
        gagg = cmul(cconj(ab), make_float2(__builtin_fmaf(cf[2 * k], gy[k], gagg.x),
                                           __builtin_fmaf(-cf[2 * k + 1], gy[k], gagg.y)));
      }
      float2 As = cconj(cexp_scaled(dsum, ps.x, ps.y));
      if constexpr (RST) As = cscale(As, lane_keep);
      const float2 gc = gcs[cl][n];
      if (j == R - 1) gagg = cfma(As, gc, gagg);       // the later chunk enters lane 15
      cplx_scan_suffix_row(As, gagg);
      // lane 0: the adjoint leaving the chunk, and the chunk's prod(conj Abar)
      if (j == 0) {
        gcs[cl][n] = gagg;
        gds[cl][n] = cmul(As, gds[cl][n]);
      }
    }
    __syncthreads();
    if (ch > ch_begin) {
      stage.store(tile, N, tid);
      __syncthreads();
    }
  }

  if (active && j == 0) {
    const int64_t k = (c * p.nseg + seg) * N;
    for (int n = 0; n < N; ++n) {
      p.seg_gloc[k + n] = gcs[cl][n];
      p.seg_gdec[k + n] = gds[cl][n];
    }
  }
}

// One thread per (channel, n): the adjoint entering segment s from the right
// is segment s + 1's G plus its prod(conj Abar) times the adjoint entering it;
// zero enters the last segment.
__global__ __launch_bounds__(256) void bwd_seg_carry_complex_kernel(const CplxBwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.nchannels * p.N) return;
  const int64_t c = i / p.N;
  const int n = (int)(i - c * p.N);
  float2 g = make_float2(0.0f, 0.0f);
  for (int64_t s = p.nseg - 1; s >= 0; --s) {
    const int64_t k = (c * p.nseg + s) * p.N + n;
    p.seg_gin[k] = g;
    g = cfma(p.seg_gdec[k], g, p.seg_gloc[k]);
  }
}

template <typename T, bool RST>
hipError_t launch_bwd_complex_main(const CplxBwdParams& p, int disc, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)(p.batch * p.groups * p.nseg)), block(kBlock);
  if (disc == 0) {
    if (vec) hipLaunchKernelGGL((scan_bwd_complex_kernel<T, true, true, RST>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((scan_bwd_complex_kernel<T, true, false, RST>), grid, block, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((scan_bwd_complex_kernel<T, false, true, RST>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((scan_bwd_complex_kernel<T, false, false, RST>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_complex(const CplxBwdParams& p, int disc, bool vec, hipStream_t s) {
  {
    const int64_t total = 4 * p.batch * p.N * p.L + 2 * p.dim * p.N + 2 * p.dim;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(cplx_bwd_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return p.reset ? launch_bwd_complex_main<T, true>(p, disc, vec, s)
                 : launch_bwd_complex_main<T, false>(p, disc, vec, s);
}

template <typename T, bool RST>
hipError_t launch_bwd_seg_summary_complex(const CplxBwdParams& p, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)(p.batch * p.groups * p.nseg)), block(kBlock);
  if (vec) hipLaunchKernelGGL((bwd_seg_summary_complex_kernel<T, true, RST>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((bwd_seg_summary_complex_kernel<T, false, RST>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t dispatch_scan_bwd_complex(const CplxBwdParams& p, int dtype, int disc, bool vec,
                                     hipStream_t s) {
  return dtype == 0 ? launch_bwd_complex<float>(p, disc, vec, s)
                    : launch_bwd_complex<bf16_t>(p, disc, vec, s);
}

hipError_t dispatch_bwd_seg_summary_complex(const CplxBwdParams& p, int dtype, bool vec,
                                            hipStream_t s) {
  if (dtype == 0)
    return p.reset ? launch_bwd_seg_summary_complex<float, true>(p, vec, s)
                   : launch_bwd_seg_summary_complex<float, false>(p, vec, s);
  return p.reset ? launch_bwd_seg_summary_complex<bf16_t, true>(p, vec, s)
                 : launch_bwd_seg_summary_complex<bf16_t, false>(p, vec, s);
}

hipError_t dispatch_bwd_seg_carry_complex(const CplxBwdParams& p, hipStream_t s) {
  const int64_t blocks = (p.nchannels * p.N + 255) / 256;
  hipLaunchKernelGGL(bwd_seg_carry_complex_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mscan

// C ABI of the selective-scan library: argument checks, launch-shape choice,
// workspace carving and dispatch to the HIP kernels.  Nothing here allocates,
// frees or synchronizes; every launch goes on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "kernels.hpp"
#include "mamba_scan.h"

namespace {

using mscan::kItems;
using mscan::kItemsBwd;

constexpr int64_t kMaxState = 64;
constexpr size_t kAlignWs = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(mamba_dtype dt) { return dt == MAMBA_F32 ? 4 : 2; }

// Whether rows of `seqlen` elements of `esize` bytes start 16-byte aligned
// (the vector-load kernels need it), without forming seqlen * esize.
bool rows_aligned16(int64_t seqlen, int esize) { return seqlen % (16 / esize) == 0; }

size_t round_up(size_t x) { return (x + kAlignWs - 1) / kAlignWs * kAlignWs; }

// Lanes per channel: enough waves to cover the 1024 SIMDs of the chip a few
// times over, without chunks much longer than the sequence.
int choose_lanes(int64_t nchannels, int64_t L, int items) {
  int r_par = 64;
  if (nchannels * 16 / 64 >= 2048) r_par = 16;
  else if (nchannels * 32 / 64 >= 2048) r_par = 32;
  int r_len = 64;
  if (L <= 16 * items) r_len = 16;
  else if (L <= 32 * items) r_len = 32;
  return r_par < r_len ? r_par : r_len;
}

bool valid_lanes(int r) { return r == 16 || r == 32 || r == 64; }

mamba_status check_sizes(mamba_dtype dt, int disc, int64_t batch, int64_t dim, int64_t dstate,
                         int64_t seqlen) {
  if (dt != MAMBA_F32 && dt != MAMBA_BF16) return MAMBA_ERR_DTYPE;
  if (disc != MAMBA_DISC_ZOH && disc != MAMBA_DISC_EULER) return MAMBA_ERR_DTYPE;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return MAMBA_ERR_SHAPE;
  if (dstate > kMaxState) return MAMBA_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 62;
  if (batch > lim / dim) return MAMBA_ERR_UNSUPPORTED;
  const int64_t nch = batch * dim;
  if (nch > lim / seqlen || nch > lim / kMaxState) return MAMBA_ERR_UNSUPPORTED;
  if (seqlen > lim / dstate || batch > lim / (dstate * seqlen)) return MAMBA_ERR_UNSUPPORTED;
  // grid sizes must fit the 32-bit grid dimension
  if (nch / 4 + 1 > (int64_t)0x7FFFFFFF) return MAMBA_ERR_UNSUPPORTED;
  return MAMBA_OK;
}

// Sequence segmentation.  When a sequence is long and its channels alone give
// too few workgroups to fill the chip, the sequence is split into segments run
// in parallel.  Forward: a summary launch (each segment's end state from zero
// and its delta sum), a carry launch (the state entering each segment) and the
// output launch.  Backward: the same for the chunk-start states, then the
// adjoint's summary and reverse carry, then the backward kernel per segment.
// Segments are whole chunks of 16 lanes x kItems steps.
constexpr int64_t kFwdChunk = 16 * kItems;

// Segment count for `blocks` workgroups (16 channels each) over `nchunks`
// chunks: none above `max_blocks`; else the power of two that gives about
// 2048 workgroups (a power of two splits power-of-two chunk counts evenly:
// uneven splits measured slower), at most one segment per chunk, and none
// when that leaves fewer than `min_seg`.
int64_t split_segments(int64_t blocks, int64_t nchunks, int64_t max_blocks, int64_t min_seg) {
  if (blocks > max_blocks) return 1;
  const int64_t want = (2048 + blocks - 1) / blocks;
  int64_t nseg = 1;
  while (nseg < want) nseg *= 2;
  if (nseg > nchunks) nseg = nchunks;
  return nseg < min_seg ? 1 : nseg;
}

// Timings on MI355X (batch 1, N = 16, bf16, ZOH) behind the two choices.
// Forward: with 64 workgroups, 4096 steps take 0.104 ms in one pass and 0.065
// ms in 16 segments, 131072 steps 5.0 ms and 1.39 ms in 64; with 256
// workgroups 16384 steps take 1.19 ms and 0.70 ms in 32; with 512 workgroups
// every split is slower (4096 steps: 0.27 ms, 0.35 ms in 8), the summary pass
// re-reading about half of what the output pass reads; 2 segments never gain,
// and sequences of 4 chunks lose in 4 (0.019 ms, 0.025 ms) and break even in 8.
int64_t auto_segments(int64_t batch, int64_t dim, int64_t seqlen) {
  const int64_t blocks = batch * mscan::channel_groups(dim, 16);
  return split_segments(blocks, (seqlen + kFwdChunk - 1) / kFwdChunk, 256, 8);
}

// Backward: heavier per chunk, so its extra passes cost relatively less.  With
// 64 workgroups 32768 steps take 5.8 ms in one pass and 1.14 ms in 32
// segments (2 segments: 4.1 ms); with 384 workgroups 4096 steps take 1.07 ms
// and 0.83 ms in 8; with 512, 1.18 ms and 1.09 ms; with 640 (and more) a split
// is slower (2048 steps: 0.66 ms, 0.70 ms in 4 or 8).
int64_t bwd_auto_segments(int64_t batch, int64_t dim, int64_t seqlen) {
  const int64_t blocks = batch * mscan::channel_groups(dim, mscan::kBwdLanes);
  return split_segments(blocks, (seqlen + kFwdChunk - 1) / kFwdChunk, 512, 2);
}

// Segments of at least this many chunks take the zero-start pass, the carry
// and the correcting pass over each segment's first chunks; shorter ones the
// summary pass, the carry and the pass from each segment's entering state.
// The correcting pass costs the chunks the entering state takes to decay
// below float32 resolution (a few chunks at the usual delta and A), so it
// only gains over the summary pass (about 0.65 of an output pass) on long
// segments.  Forward at batch 1, D 1024, 32 segments, zero-start scheme
// against summary pass: 4 chunks per segment 0.27 / 0.21 ms, 8 chunks 0.46 /
// 0.41 ms, 16 chunks 0.72 / 0.72 ms, 128 chunks 3.7 / 5.6 ms.
constexpr int64_t kLongSegmentChunks = 16;

// Forward workspace (segmented only): the segment end states and the
// entering states (nchannels, nseg, dstate) float32, then the delta sums and
// the reset-free factors (nchannels, nseg) float32.
struct FwdLayout {
  int64_t nseg, seg_chunks;
  size_t off_h0, off_dsum, off_keep, total;
};

FwdLayout fwd_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                     int64_t segments) {
  FwdLayout w = {1, 0, 0, 0, 0, 0};
  const int64_t nchunks = (seqlen + kFwdChunk - 1) / kFwdChunk;
  int64_t nseg = segments < nchunks ? segments : nchunks;
  if (nseg <= 1) return w;
  w.seg_chunks = (nchunks + nseg - 1) / nseg;
  w.nseg = (nchunks + w.seg_chunks - 1) / w.seg_chunks;
  if (w.nseg <= 1) return FwdLayout{1, 0, 0, 0, 0, 0};
  const size_t nst = (size_t)(batch * dim) * (size_t)w.nseg * (size_t)dstate * 4;
  const size_t nsc = round_up((size_t)(batch * dim) * (size_t)w.nseg * 4);
  w.off_h0 = round_up(nst);
  w.off_dsum = w.off_h0 + round_up(nst);
  w.off_keep = w.off_dsum + nsc;
  w.total = w.off_keep + nsc;
  return w;
}

// Backward workspace: the chunk-start states (nchannels, nchunks, dstate)
// float32, then one int flag per block, then (segmented runs only) the
// forward's segment buffers (end states from zero, entering states,
// (nchannels, nseg, dstate) each; delta sums and reset-free factors,
// (nchannels, nseg) each) and the same four for the adjoint (summaries from
// a zero end, entering adjoints, delta sums, factors).  Segments are whole
// 128-step chunks, as in the forward, with a choice of their own
// (bwd_auto_segments).
struct BwdLayout {
  int64_t nchunks, groups, nseg, seg_chunks;
  size_t off_flags, off_seg, total;
};

BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                     int64_t segments = 1) {
  BwdLayout w;
  const int64_t tch = (int64_t)mscan::kBwdLanes * kItemsBwd;
  static_assert(mscan::kBwdLanes * kItemsBwd == kFwdChunk, "forward and backward chunks agree");
  w.nchunks = (seqlen + tch - 1) / tch;
  w.groups = mscan::channel_groups(dim, mscan::kBwdLanes);
  w.nseg = 1;
  w.seg_chunks = 0;
  const int64_t want = segments < w.nchunks ? segments : w.nchunks;
  if (want > 1) {
    const int64_t sc = (w.nchunks + want - 1) / want;
    const int64_t ns = (w.nchunks + sc - 1) / sc;
    if (ns > 1) {
      w.nseg = ns;
      w.seg_chunks = sc;
    }
  }
  w.off_flags = round_up((size_t)(batch * dim) * (size_t)w.nchunks * (size_t)dstate * 4);
  w.off_seg = w.off_flags + round_up((size_t)(batch * w.groups) * (size_t)w.nseg * 4);
  w.total = w.off_seg;
  if (w.nseg > 1) {
    const size_t nst = round_up((size_t)(batch * dim) * (size_t)w.nseg * (size_t)dstate * 4);
    const size_t nsc = round_up((size_t)(batch * dim) * (size_t)w.nseg * 4);
    w.total += 4 * nst + 4 * nsc;
  }
  return w;
}

// The segment buffers of a segmented backward, from `q` (offset w.off_seg of
// the layout).
struct BwdSegBuffers {
  float *h_end, *h_in, *dsum, *keep, *g_loc, *g_in, *g_dsum, *g_keep;
};

BwdSegBuffers bwd_seg_buffers(const BwdLayout& w, int64_t nchannels, int64_t dstate, char* q) {
  const size_t nst = round_up((size_t)nchannels * (size_t)w.nseg * (size_t)dstate * 4);
  const size_t nsc = round_up((size_t)nchannels * (size_t)w.nseg * 4);
  BwdSegBuffers s;
  s.h_end = reinterpret_cast<float*>(q);
  s.h_in = reinterpret_cast<float*>(q + nst);
  s.g_loc = reinterpret_cast<float*>(q + 2 * nst);
  s.g_in = reinterpret_cast<float*>(q + 3 * nst);
  s.dsum = reinterpret_cast<float*>(q + 4 * nst);
  s.keep = reinterpret_cast<float*>(q + 4 * nst + nsc);
  s.g_dsum = reinterpret_cast<float*>(q + 4 * nst + 2 * nsc);
  s.g_keep = reinterpret_cast<float*>(q + 4 * nst + 3 * nsc);
  return s;
}

// Complex workspaces (complex float32 = 8 bytes).  Forward (segmented only):
// per channel, segment and state the end state from zero, the entering state
// and prod(Abar).  Backward: the chunk-start states (unless the forward's
// checkpoints are given), then, segmented, the same three buffers for the
// state pass and three for the adjoint (G from a zero end, the entering
// adjoint, prod(conj Abar)).  Segments as in the real calls.
struct CplxLayout {
  int64_t nchunks, groups, nseg, seg_chunks;
  size_t off_seg, nst, total;
};

CplxLayout cplx_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                       int64_t segments, bool bwd) {
  const BwdLayout b = bwd_layout(batch, dim, dstate, seqlen, segments);
  CplxLayout w;
  w.nchunks = b.nchunks;
  w.groups = b.groups;
  w.nseg = b.nseg;
  w.seg_chunks = b.seg_chunks;
  w.off_seg = bwd ? round_up((size_t)(batch * dim) * (size_t)w.nchunks * (size_t)dstate * 8) : 0;
  w.nst = round_up((size_t)(batch * dim) * (size_t)w.nseg * (size_t)dstate * 8);
  w.total = w.off_seg + (w.nseg > 1 ? (bwd ? 6 : 3) * w.nst : 0);
  return w;
}

inline mamba_status hip_status(hipError_t e) { return e == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP; }

}  // namespace

extern "C" {

int mamba_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

const char* mamba_status_string(mamba_status s) {
  switch (s) {
    case MAMBA_OK: return "ok";
    case MAMBA_ERR_NULL_PTR: return "a required pointer is NULL";
    case MAMBA_ERR_SHAPE: return "a size is zero or negative";
    case MAMBA_ERR_DTYPE: return "unknown dtype or discretization";
    case MAMBA_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case MAMBA_ERR_WORKSPACE: return "workspace missing or too small";
    case MAMBA_ERR_UNSUPPORTED: return "sizes outside the supported limits";
    case MAMBA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case MAMBA_ERR_INVALID: return "inconsistent optional arguments";
    case MAMBA_ERR_SCRATCH_LIMIT:
      return "the problem needs more scratch than the allocation-free entry point's fixed "
             "device array holds";
  }
  return "unknown status";
}

size_t mamba_scan_fwd_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                        int64_t seqlen, mamba_dtype dt, int lanes_per_channel,
                                        int segments) {
  if (check_sizes(dt, MAMBA_DISC_ZOH, batch, dim, dstate, seqlen) != MAMBA_OK) return SIZE_MAX;
  if (segments < 0) return SIZE_MAX;
  const int64_t want = segments != 0 ? segments
                       : (lanes_per_channel != 0 && lanes_per_channel != 16)
                           ? 1   // an explicit wider lane layout runs in one pass
                           : auto_segments(batch, dim, seqlen);
  const FwdLayout w = fwd_layout(batch, dim, dstate, seqlen, want);
  if (w.nseg > 1 && lanes_per_channel != 0 && lanes_per_channel != 16) return SIZE_MAX;
  return w.total;
}

size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                     mamba_dtype dt) {
  return mamba_scan_fwd_workspace_size_ex(batch, dim, dstate, seqlen, dt, 0, 0);
}

// Workspace of mamba_scan_bwd_ex for a lanes-per-channel and segments
// choice.  The backward always spreads a channel over 16 lanes: 0 and 16 are
// accepted.
size_t mamba_scan_bwd_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                        mamba_dtype dt, int lanes_per_channel, int segments) {
  if (check_sizes(dt, MAMBA_DISC_ZOH, batch, dim, dstate, seqlen) != MAMBA_OK) return SIZE_MAX;
  if (lanes_per_channel != 0 && lanes_per_channel != mscan::kBwdLanes) return SIZE_MAX;
  if (segments < 0) return SIZE_MAX;
  const int64_t want = segments != 0 ? segments : bwd_auto_segments(batch, dim, seqlen);
  return bwd_layout(batch, dim, dstate, seqlen, want).total;
}

size_t mamba_scan_checkpoint_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  if (check_sizes(MAMBA_F32, MAMBA_DISC_ZOH, batch, dim, dstate, seqlen) != MAMBA_OK)
    return SIZE_MAX;
  const BwdLayout w = bwd_layout(batch, dim, dstate, seqlen);
  return (size_t)(batch * dim) * (size_t)w.nchunks * (size_t)dstate * 4;
}

size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                     mamba_dtype dt) {
  return mamba_scan_bwd_workspace_size_ex(batch, dim, dstate, seqlen, dt, 0, 0);
}

// Same as mamba_scan_fwd with an explicit lanes-per-channel choice (16, 32 or
// 64; 0 = automatic).  For tests and tuning.
mamba_status mamba_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                               const void* C, const float* D, const void* z,
                               const float* delta_bias, const float* h0, const uint8_t* reset,
                               int delta_softplus,
                               mamba_disc disc, mamba_dtype dt, int64_t batch, int64_t dim,
                               int64_t dstate, int64_t seqlen, void* out, float* last_state,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int lanes_per_channel, int segments, float* checkpoints,
                               void* timing_begin, void* timing_end) {
  mamba_status st = check_sizes(dt, disc, batch, dim, dstate, seqlen);
  if (st != MAMBA_OK) return st;
  if (!u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL_PTR;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, out, last_state, workspace,
                        checkpoints};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MAMBA_ERR_ALIGNMENT;
  if (segments < 0) return MAMBA_ERR_UNSUPPORTED;
  const int64_t want = segments != 0 ? segments
                       : (lanes_per_channel != 0 && lanes_per_channel != 16)
                           ? 1   // an explicit wider lane layout runs in one pass
                           : auto_segments(batch, dim, seqlen);
  const FwdLayout w = fwd_layout(batch, dim, dstate, seqlen, want);
  bool segmented = w.nseg > 1;
  if (segmented) {
    if (lanes_per_channel != 0 && lanes_per_channel != 16) return MAMBA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < w.total) {
      if (segments != 0) return MAMBA_ERR_WORKSPACE;
      segmented = false;   // automatic choice without the workspace: one pass
    }
  }
  // reset flags and checkpoints (128-step chunks) run with 16 lanes per channel
  if ((reset || checkpoints) && lanes_per_channel != 0 && lanes_per_channel != 16)
    return MAMBA_ERR_UNSUPPORTED;
  int lanes = (segmented || reset || checkpoints) ? 16 : lanes_per_channel;
  if (lanes == 0) lanes = choose_lanes(batch * dim, seqlen, kItems);
  if (!valid_lanes(lanes)) return MAMBA_ERR_UNSUPPORTED;

  mscan::FwdParams p;
  memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.bias = delta_bias;
  p.h0 = h0; p.out = out; p.last_state = last_state; p.chunk_states = checkpoints;
  p.reset = reset;
  p.batch = batch; p.dim = dim; p.L = seqlen; p.nchannels = batch * dim;
  p.groups = mscan::channel_groups(dim, lanes);
  p.N = (int)dstate; p.softplus = delta_softplus ? 1 : 0;
  p.nseg = 1;
  p.seg_chunks = 0;
  if (batch * p.groups > (int64_t)0x7FFFFFFF / w.nseg) return MAMBA_ERR_UNSUPPORTED;
  const bool vec = rows_aligned16(seqlen, elem_size(dt));
  const int dti = dt == MAMBA_F32 ? 0 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool long_seg = segmented && w.seg_chunks >= kLongSegmentChunks;
  if (segmented) {
    // long segments: every segment from zero (with its summary), the carry,
    // then each segment's first chunks again from its entering state; short
    // ones: the summaries, the carry, then every segment from its entering
    // state
    char* ws = static_cast<char*>(workspace);
    p.nseg = w.nseg;
    p.seg_chunks = w.seg_chunks;
    p.seg_state = reinterpret_cast<float*>(ws);
    p.seg_h0 = reinterpret_cast<float*>(ws + w.off_h0);
    p.seg_dsum = reinterpret_cast<float*>(ws + w.off_dsum);
    p.seg_keep = reinterpret_cast<float*>(ws + w.off_keep);
    if (long_seg) {
      p.seg_pass = mscan::kSegLocal;
    } else {
      if (mscan::dispatch_seg_summary(p, dti, (int)disc, vec, s) != hipSuccess)
        return MAMBA_ERR_HIP;
      if (mscan::dispatch_seg_carry(p, s) != hipSuccess) return MAMBA_ERR_HIP;
    }
  }
  if (timing_begin && hipEventRecord(static_cast<hipEvent_t>(timing_begin), s) != hipSuccess)
    return MAMBA_ERR_HIP;
  if (mscan::dispatch_scan_fwd(p, dti, (int)disc, lanes, vec, s) != hipSuccess)
    return MAMBA_ERR_HIP;
  if (timing_end && hipEventRecord(static_cast<hipEvent_t>(timing_end), s) != hipSuccess)
    return MAMBA_ERR_HIP;
  if (segmented && long_seg) {
    if (mscan::dispatch_seg_carry(p, s) != hipSuccess) return MAMBA_ERR_HIP;
    if (mscan::dispatch_scan_fwd_fix(p, dti, (int)disc, vec, s) != hipSuccess)
      return MAMBA_ERR_HIP;
  }
  return MAMBA_OK;
}

mamba_status mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z,
                            const float* delta_bias, const float* h0, int delta_softplus,
                            mamba_disc disc, mamba_dtype dt, int64_t batch, int64_t dim,
                            int64_t dstate, int64_t seqlen, void* out, float* last_state,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return mamba_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, nullptr, delta_softplus,
                           disc, dt, batch, dim, dstate, seqlen, out, last_state, workspace,
                           workspace_bytes, stream, 0, 0, nullptr, nullptr, nullptr);
}

mamba_status mamba_scan_fwd_varlen(const void* u, const void* delta, const float* A,
                                   const void* B, const void* C, const float* D, const void* z,
                                   const float* delta_bias, const float* h0,
                                   const uint8_t* reset, int delta_softplus, mamba_disc disc,
                                   mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                   int64_t seqlen, void* out, float* last_state, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!reset) return MAMBA_ERR_NULL_PTR;
  return mamba_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, reset, delta_softplus, disc,
                           dt, batch, dim, dstate, seqlen, out, last_state, workspace,
                           workspace_bytes, stream, 0, 0, nullptr, nullptr, nullptr);
}

mamba_status mamba_scan_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                               const void* C, const float* D, const void* z,
                               const float* delta_bias, const float* h0, const void* dout,
                               const uint8_t* reset, int delta_softplus, mamba_disc disc,
                               mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                               int64_t seqlen, float* du, float* ddelta, float* dA, float* dB,
                               float* dC, float* dD, float* dz, float* ddelta_bias, float* dh0,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int lanes_per_channel, int segments, const float* checkpoints,
                               void* timing_begin, void* timing_end) {
  mamba_status st = check_sizes(dt, disc, batch, dim, dstate, seqlen);
  if (st != MAMBA_OK) return st;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
    return MAMBA_ERR_NULL_PTR;
  if ((D == nullptr) != (dD == nullptr) || (z == nullptr) != (dz == nullptr) ||
      (delta_bias == nullptr) != (ddelta_bias == nullptr) || (h0 == nullptr && dh0 != nullptr))
    return MAMBA_ERR_INVALID;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, dout, du, ddelta, dA, dB, dC,
                        dD, dz, ddelta_bias, dh0, workspace, checkpoints};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MAMBA_ERR_ALIGNMENT;
  if (lanes_per_channel != 0 && lanes_per_channel != mscan::kBwdLanes) return MAMBA_ERR_UNSUPPORTED;
  const int lanes = mscan::kBwdLanes;
  if (segments < 0) return MAMBA_ERR_UNSUPPORTED;
  const int64_t want = segments != 0 ? segments : bwd_auto_segments(batch, dim, seqlen);
  BwdLayout w = bwd_layout(batch, dim, dstate, seqlen, want);
  // with checkpoints from the forward only the part past the states is used
  size_t need = checkpoints ? w.total - w.off_flags : w.total;
  if (w.nseg > 1 && (!workspace || workspace_bytes < need)) {
    if (segments != 0) return MAMBA_ERR_WORKSPACE;
    w = bwd_layout(batch, dim, dstate, seqlen);   // automatic choice without the room: one pass
    need = checkpoints ? w.total - w.off_flags : w.total;
  }
  if (!workspace || workspace_bytes < need) return MAMBA_ERR_WORKSPACE;
  if (batch * w.groups > (int64_t)0x7FFFFFFF / w.nseg) return MAMBA_ERR_UNSUPPORTED;

  float* states = checkpoints ? const_cast<float*>(checkpoints) : static_cast<float*>(workspace);
  // with checkpoints the workspace starts at the flags
  char* flags = static_cast<char*>(workspace) + (checkpoints ? 0 : w.off_flags);
  const bool segmented = w.nseg > 1;
  BwdSegBuffers sb;
  memset(&sb, 0, sizeof(sb));
  if (segmented) sb = bwd_seg_buffers(w, batch * dim, dstate, flags + (w.off_seg - w.off_flags));
  const bool vec = rows_aligned16(seqlen, elem_size(dt));
  const int dti = dt == MAMBA_F32 ? 0 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);

  mscan::FwdParams fp;
  memset(&fp, 0, sizeof(fp));
  fp.u = u; fp.delta = delta; fp.A = A; fp.B = B; fp.C = C; fp.D = D; fp.z = z;
  fp.bias = delta_bias; fp.h0 = h0; fp.out = nullptr; fp.last_state = nullptr;
  fp.chunk_states = states;
  fp.reset = reset;
  fp.batch = batch; fp.dim = dim; fp.L = seqlen; fp.nchannels = batch * dim;
  fp.groups = w.groups;
  fp.nseg = 1;
  fp.seg_chunks = 0;
  fp.N = (int)dstate; fp.softplus = delta_softplus ? 1 : 0;
  if (!checkpoints) {
    // the states at every chunk start, segment by segment, in the forward's
    // two schemes
    const bool long_seg = segmented && w.seg_chunks >= kLongSegmentChunks;
    if (segmented) {
      fp.nseg = w.nseg;
      fp.seg_chunks = w.seg_chunks;
      fp.seg_state = sb.h_end;
      fp.seg_h0 = sb.h_in;
      fp.seg_dsum = sb.dsum;
      fp.seg_keep = sb.keep;
      if (long_seg) {
        fp.seg_pass = mscan::kSegLocal;
      } else {
        if (mscan::dispatch_seg_summary(fp, dti, (int)disc, vec, s) != hipSuccess)
          return MAMBA_ERR_HIP;
        if (mscan::dispatch_seg_carry(fp, s) != hipSuccess) return MAMBA_ERR_HIP;
      }
    }
    if (mscan::dispatch_chunk_states(fp, dti, (int)disc, lanes, vec, s) != hipSuccess)
      return MAMBA_ERR_HIP;
    if (long_seg) {
      if (mscan::dispatch_seg_carry(fp, s) != hipSuccess) return MAMBA_ERR_HIP;
      if (mscan::dispatch_chunk_states_fix(fp, dti, (int)disc, vec, s) != hipSuccess)
        return MAMBA_ERR_HIP;
    }
  }

  mscan::BwdParams p;
  memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.bias = delta_bias;
  p.h0 = h0; p.dout = dout; p.du = du; p.ddelta = ddelta; p.dA = dA; p.dB = dB; p.dC = dC;
  p.dD = dD; p.dz = dz; p.dbias = ddelta_bias; p.dh0 = dh0;
  p.chunk_states = states;
  p.reset = reset;
  p.deferred = reinterpret_cast<int*>(flags);
  p.batch = batch; p.dim = dim; p.L = seqlen; p.nchannels = batch * dim;
  p.nchunks = w.nchunks; p.groups = w.groups; p.N = (int)dstate;
  p.softplus = delta_softplus ? 1 : 0;
  p.nseg = w.nseg;
  p.seg_chunks = w.seg_chunks;
  if (segmented) {
    p.seg_gloc = sb.g_loc;
    p.seg_gdsum = sb.g_dsum;
    p.seg_gkeep = sb.g_keep;
    p.seg_gin = sb.g_in;
    if (mscan::dispatch_bwd_seg_summary(p, dti, vec, s) != hipSuccess) return MAMBA_ERR_HIP;
    if (mscan::dispatch_bwd_seg_carry(p, s) != hipSuccess) return MAMBA_ERR_HIP;
  }
  return hip_status(mscan::dispatch_scan_bwd(p, dti, (int)disc, vec, s,
                                             static_cast<hipEvent_t>(timing_begin),
                                             static_cast<hipEvent_t>(timing_end)));
}

mamba_status mamba_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z,
                            const float* delta_bias, const float* h0, const void* dout,
                            int delta_softplus, mamba_disc disc, mamba_dtype dt, int64_t batch,
                            int64_t dim, int64_t dstate, int64_t seqlen, float* du,
                            float* ddelta, float* dA, float* dB, float* dC, float* dD, float* dz,
                            float* ddelta_bias, float* dh0, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return mamba_scan_bwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, dout, nullptr,
                           delta_softplus, disc, dt, batch, dim, dstate, seqlen, du, ddelta, dA,
                           dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes, stream, 0,
                           0, nullptr, nullptr, nullptr);
}

mamba_status mamba_scan_bwd_varlen(const void* u, const void* delta, const float* A,
                                   const void* B, const void* C, const float* D, const void* z,
                                   const float* delta_bias, const float* h0, const void* dout,
                                   const uint8_t* reset, int delta_softplus, mamba_disc disc,
                                   mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                   int64_t seqlen, float* du, float* ddelta, float* dA,
                                   float* dB, float* dC, float* dD, float* dz,
                                   float* ddelta_bias, float* dh0, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!reset) return MAMBA_ERR_NULL_PTR;
  return mamba_scan_bwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, dout, reset, delta_softplus,
                           disc, dt, batch, dim, dstate, seqlen, du, ddelta, dA, dB, dC, dD, dz,
                           ddelta_bias, dh0, workspace, workspace_bytes, stream, 0, 0, nullptr,
                           nullptr, nullptr);
}

mamba_status mamba_state_update(float* state, const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, int delta_softplus, mamba_disc disc,
                                mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                void* out, void* stream) {
  mamba_status st = check_sizes(dt, disc, batch, dim, dstate, 1);
  if (st != MAMBA_OK) return st;
  if (!state || !u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL_PTR;
  const void* ptrs[] = {state, u, delta, A, B, C, D, z, delta_bias, out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MAMBA_ERR_ALIGNMENT;
  mscan::StepParams p;
  memset(&p, 0, sizeof(p));
  p.state = state; p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.bias = delta_bias; p.out = out; p.batch = batch; p.dim = dim; p.nchannels = batch * dim;
  p.N = (int)dstate; p.softplus = delta_softplus ? 1 : 0;
  return hip_status(mscan::dispatch_state_update(p, dt == MAMBA_F32 ? 0 : 1, (int)disc,
                                                 static_cast<hipStream_t>(stream)));
}

// ---- complex-valued decode step ----
mamba_status mamba_state_update_complex(float* state, const void* u, const void* delta,
                                        const float* A, const float* B, const float* C,
                                        const float* D, const void* z, const float* delta_bias,
                                        int delta_softplus, mamba_disc disc, mamba_dtype dt,
                                        int64_t batch, int64_t dim, int64_t dstate, void* out,
                                        void* stream) {
  mamba_status st = check_sizes(dt, disc, batch, dim, dstate, 1);
  if (st != MAMBA_OK) return st;
  if (dstate > 16) return MAMBA_ERR_UNSUPPORTED;
  if (!state || !u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL_PTR;
  const void* ptrs[] = {state, u, delta, A, B, C, D, z, delta_bias, out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_ALIGNMENT;
  mscan::CplxStepParams p;
  memset(&p, 0, sizeof(p));
  p.state = reinterpret_cast<float2*>(state); p.u = u; p.delta = delta;
  p.A = reinterpret_cast<const float2*>(A); p.B = reinterpret_cast<const float2*>(B);
  p.C = reinterpret_cast<const float2*>(C); p.D = D; p.z = z; p.bias = delta_bias; p.out = out;
  p.batch = batch; p.dim = dim; p.nchannels = batch * dim;
  p.N = (int)dstate; p.softplus = delta_softplus ? 1 : 0;
  return hip_status(mscan::dispatch_state_update_complex(p, dt == MAMBA_F32 ? 0 : 1, (int)disc,
                                                         static_cast<hipStream_t>(stream)));
}

// ---- complex-valued forward ----
size_t mamba_scan_complex_checkpoint_size(int64_t batch, int64_t dim, int64_t dstate,
                                          int64_t seqlen) {
  if (check_sizes(MAMBA_F32, MAMBA_DISC_ZOH, batch, dim, dstate, seqlen) != MAMBA_OK ||
      dstate > 16)
    return SIZE_MAX;
  const BwdLayout w = bwd_layout(batch, dim, dstate, seqlen);
  return (size_t)(batch * dim) * (size_t)w.nchunks * (size_t)dstate * 8;
}

size_t mamba_scan_fwd_complex_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                                int64_t seqlen, int segments) {
  if (check_sizes(MAMBA_F32, MAMBA_DISC_ZOH, batch, dim, dstate, seqlen) != MAMBA_OK ||
      dstate > 16 || segments < 0)
    return SIZE_MAX;
  const int64_t want = segments != 0 ? segments : auto_segments(batch, dim, seqlen);
  return cplx_layout(batch, dim, dstate, seqlen, want, false).total;
}

size_t mamba_scan_fwd_complex_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                             int64_t seqlen) {
  return mamba_scan_fwd_complex_workspace_size_ex(batch, dim, dstate, seqlen, 0);
}

mamba_status mamba_scan_fwd_complex(const void* u, const void* delta, const float* A,
                                    const float* B, const float* C, const float* D,
                                    const void* z, const float* delta_bias, const float* h0,
                                    int delta_softplus, mamba_disc disc, mamba_dtype dt,
                                    int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                    void* out, float* last_state, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return mamba_scan_fwd_complex_ex(u, delta, A, B, C, D, z, delta_bias, h0, nullptr,
                                   delta_softplus, disc, dt, batch, dim, dstate, seqlen, out,
                                   last_state, nullptr, workspace, workspace_bytes, stream, 0);
}

mamba_status mamba_scan_fwd_complex_ex(const void* u, const void* delta, const float* A,
                                       const float* B, const float* C, const float* D,
                                       const void* z, const float* delta_bias, const float* h0,
                                       const uint8_t* reset, int delta_softplus, mamba_disc disc,
                                       mamba_dtype dt,
                                       int64_t batch, int64_t dim, int64_t dstate,
                                       int64_t seqlen, void* out, float* last_state,
                                       float* checkpoints, void* workspace,
                                       size_t workspace_bytes, void* stream, int segments) {
  mamba_status st = check_sizes(dt, disc, batch, dim, dstate, seqlen);
  if (st != MAMBA_OK) return st;
  if (dstate > 16 || segments < 0) return MAMBA_ERR_UNSUPPORTED;
  if (!u || !delta || !A || !B || !C || !out) return MAMBA_ERR_NULL_PTR;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, out, last_state, checkpoints,
                        workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_ALIGNMENT;
  const int64_t want = segments != 0 ? segments : auto_segments(batch, dim, seqlen);
  CplxLayout w = cplx_layout(batch, dim, dstate, seqlen, want, false);
  bool segmented = w.nseg > 1;
  if (segmented && (!workspace || workspace_bytes < w.total)) {
    if (segments != 0) return MAMBA_ERR_WORKSPACE;
    segmented = false;   // automatic choice without the workspace: one pass
    w = cplx_layout(batch, dim, dstate, seqlen, 1, false);
  }
  mscan::CplxParams p;
  memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.A = reinterpret_cast<const float2*>(A);
  p.B = reinterpret_cast<const float2*>(B); p.C = reinterpret_cast<const float2*>(C);
  p.D = D; p.z = z; p.bias = delta_bias; p.h0 = reinterpret_cast<const float2*>(h0);
  p.out = out; p.last_state = reinterpret_cast<float2*>(last_state);
  p.chunk_states = reinterpret_cast<float2*>(checkpoints);
  p.reset = reset;
  p.batch = batch; p.dim = dim; p.L = seqlen; p.nchannels = batch * dim;
  p.groups = w.groups;
  p.nseg = 1;
  p.N = (int)dstate; p.softplus = delta_softplus ? 1 : 0;
  if (batch * p.groups > (int64_t)0x7FFFFFFF / w.nseg) return MAMBA_ERR_UNSUPPORTED;
  const bool vec = rows_aligned16(seqlen, elem_size(dt));
  const int dti = dt == MAMBA_F32 ? 0 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (segmented) {
    // the summaries (each segment from zero), the carry (also the last
    // state), then every segment from its entering state
    char* ws = static_cast<char*>(workspace);
    p.nseg = w.nseg;
    p.seg_chunks = w.seg_chunks;
    p.seg_state = reinterpret_cast<float2*>(ws);
    p.seg_h0 = reinterpret_cast<float2*>(ws + w.nst);
    p.seg_dec = reinterpret_cast<float2*>(ws + 2 * w.nst);
    if (mscan::dispatch_seg_summary_complex(p, dti, (int)disc, vec, s) != hipSuccess)
      return MAMBA_ERR_HIP;
    if (mscan::dispatch_seg_carry_complex(p, s) != hipSuccess) return MAMBA_ERR_HIP;
  }
  return hip_status(mscan::dispatch_scan_fwd_complex(p, dti, (int)disc, vec, s));
}

size_t mamba_scan_bwd_complex_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                                int64_t seqlen, int segments) {
  if (check_sizes(MAMBA_F32, MAMBA_DISC_ZOH, batch, dim, dstate, seqlen) != MAMBA_OK ||
      dstate > 16 || segments < 0)
    return SIZE_MAX;
  const int64_t want = segments != 0 ? segments : bwd_auto_segments(batch, dim, seqlen);
  return cplx_layout(batch, dim, dstate, seqlen, want, true).total;
}

size_t mamba_scan_bwd_complex_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                             int64_t seqlen) {
  return mamba_scan_bwd_complex_workspace_size_ex(batch, dim, dstate, seqlen, 0);
}

mamba_status mamba_scan_bwd_complex(const void* u, const void* delta, const float* A,
                                    const float* B, const float* C, const float* D,
                                    const void* z, const float* delta_bias, const float* h0,
                                    const void* dout, int delta_softplus, mamba_disc disc,
                                    mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                    int64_t seqlen, float* du, float* ddelta, float* dA,
                                    float* dB, float* dC, float* dD, float* dz,
                                    float* ddelta_bias, float* dh0, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return mamba_scan_bwd_complex_ex(u, delta, A, B, C, D, z, delta_bias, h0, dout, nullptr,
                                   delta_softplus, disc, dt, batch, dim, dstate, seqlen, du,
                                   ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, nullptr,
                                   workspace, workspace_bytes, stream, 0);
}

mamba_status mamba_scan_bwd_complex_ex(const void* u, const void* delta, const float* A,
                                       const float* B, const float* C, const float* D,
                                       const void* z, const float* delta_bias, const float* h0,
                                       const void* dout, const uint8_t* reset,
                                       int delta_softplus, mamba_disc disc,
                                       mamba_dtype dt, int64_t batch, int64_t dim,
                                       int64_t dstate, int64_t seqlen, float* du, float* ddelta,
                                       float* dA, float* dB, float* dC, float* dD, float* dz,
                                       float* ddelta_bias, float* dh0, const float* checkpoints,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       int segments) {
  mamba_status st = check_sizes(dt, disc, batch, dim, dstate, seqlen);
  if (st != MAMBA_OK) return st;
  if (dstate > 16 || segments < 0) return MAMBA_ERR_UNSUPPORTED;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
    return MAMBA_ERR_NULL_PTR;
  if ((D == nullptr) != (dD == nullptr) || (z == nullptr) != (dz == nullptr) ||
      (delta_bias == nullptr) != (ddelta_bias == nullptr) || (h0 == nullptr && dh0 != nullptr))
    return MAMBA_ERR_INVALID;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, dout, du, ddelta, dA, dB, dC,
                        dD, dz, ddelta_bias, dh0, workspace, checkpoints};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_ALIGNMENT;
  const int64_t want = segments != 0 ? segments : bwd_auto_segments(batch, dim, seqlen);
  CplxLayout w = cplx_layout(batch, dim, dstate, seqlen, want, true);
  // with checkpoints the chunk-start states are not in the workspace
  size_t need = checkpoints ? w.total - w.off_seg : w.total;
  if (w.nseg > 1 && (!workspace || workspace_bytes < need)) {
    if (segments != 0) return MAMBA_ERR_WORKSPACE;
    w = cplx_layout(batch, dim, dstate, seqlen, 1, true);   // automatic: one pass
    need = checkpoints ? w.total - w.off_seg : w.total;
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return MAMBA_ERR_WORKSPACE;
  if (batch * w.groups > (int64_t)0x7FFFFFFF / w.nseg) return MAMBA_ERR_UNSUPPORTED;
  const bool segmented = w.nseg > 1;
  const bool vec = rows_aligned16(seqlen, elem_size(dt));
  const int dti = dt == MAMBA_F32 ? 0 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* states = checkpoints ? reinterpret_cast<float2*>(const_cast<float*>(checkpoints))
                               : static_cast<float2*>(workspace);
  char* segbase = segmented ? static_cast<char*>(workspace) + (checkpoints ? 0 : w.off_seg)
                            : nullptr;
  auto seg_buf = [&](int i) { return reinterpret_cast<float2*>(segbase + i * w.nst); };

  mscan::CplxParams fp;
  memset(&fp, 0, sizeof(fp));
  fp.u = u; fp.delta = delta; fp.A = reinterpret_cast<const float2*>(A);
  fp.B = reinterpret_cast<const float2*>(B); fp.C = reinterpret_cast<const float2*>(C);
  fp.D = D; fp.z = z; fp.bias = delta_bias; fp.h0 = reinterpret_cast<const float2*>(h0);
  fp.chunk_states = states;
  fp.reset = reset;
  fp.batch = batch; fp.dim = dim; fp.L = seqlen; fp.nchannels = batch * dim;
  fp.groups = w.groups; fp.N = (int)dstate; fp.softplus = delta_softplus ? 1 : 0;
  fp.nseg = 1;
  if (!checkpoints) {
    if (segmented) {
      // the states at every chunk start, segment by segment: summaries,
      // carry, then every segment from its entering state
      fp.nseg = w.nseg;
      fp.seg_chunks = w.seg_chunks;
      fp.seg_state = seg_buf(0);
      fp.seg_h0 = seg_buf(1);
      fp.seg_dec = seg_buf(2);
      if (mscan::dispatch_seg_summary_complex(fp, dti, (int)disc, vec, s) != hipSuccess)
        return MAMBA_ERR_HIP;
      if (mscan::dispatch_seg_carry_complex(fp, s) != hipSuccess) return MAMBA_ERR_HIP;
    }
    if (mscan::dispatch_chunk_states_complex(fp, dti, (int)disc, vec, s) != hipSuccess)
      return MAMBA_ERR_HIP;
  }

  mscan::CplxBwdParams p;
  memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.A = fp.A; p.B = fp.B; p.C = fp.C; p.D = D; p.z = z;
  p.bias = delta_bias; p.h0 = fp.h0; p.dout = dout; p.du = du; p.ddelta = ddelta;
  p.dA = reinterpret_cast<float2*>(dA); p.dB = reinterpret_cast<float2*>(dB);
  p.dC = reinterpret_cast<float2*>(dC); p.dD = dD; p.dz = dz; p.dbias = ddelta_bias;
  p.dh0 = reinterpret_cast<float2*>(dh0); p.chunk_states = states;
  p.reset = reset;
  p.batch = batch; p.dim = dim; p.L = seqlen; p.nchannels = batch * dim;
  p.nchunks = w.nchunks; p.groups = w.groups; p.N = (int)dstate;
  p.softplus = delta_softplus ? 1 : 0;
  p.nseg = w.nseg;
  p.seg_chunks = w.seg_chunks;
  if (segmented) {
    p.seg_gloc = seg_buf(3);
    p.seg_gin = seg_buf(4);
    p.seg_gdec = seg_buf(5);
    if (mscan::dispatch_bwd_seg_summary_complex(p, dti, vec, s) != hipSuccess)
      return MAMBA_ERR_HIP;
    if (mscan::dispatch_bwd_seg_carry_complex(p, s) != hipSuccess) return MAMBA_ERR_HIP;
  }
  return hip_status(mscan::dispatch_scan_bwd_complex(p, dti, (int)disc, vec, s));
}

// ---- short causal convolution + SiLU ----
mamba_status mamba_conv1d_silu_fwd(const void* x, const float* w, const float* b,
                                   const uint8_t* reset, int64_t width, mamba_dtype dt,
                                   int64_t batch, int64_t dim, int64_t seqlen, void* u,
                                   void* stream) {
  mamba_status st = check_sizes(dt, MAMBA_DISC_ZOH, batch, dim, 1, seqlen);
  if (st != MAMBA_OK) return st;
  if (width < 1 || width > 4) return MAMBA_ERR_UNSUPPORTED;
  if (!x || !w || !u) return MAMBA_ERR_NULL_PTR;
  const void* ptrs[] = {x, w, b, u};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_ALIGNMENT;
  mscan::ConvParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.w = w; p.b = b; p.reset = reset; p.u = u;
  p.batch = batch; p.dim = dim; p.L = seqlen; p.nchannels = batch * dim;
  p.tiles = mscan::conv_tiles(seqlen); p.W = (int)width;
  if (p.nchannels * p.tiles > (int64_t)0x7FFFFFFF) return MAMBA_ERR_UNSUPPORTED;
  const bool vec = rows_aligned16(seqlen, elem_size(dt));
  return hip_status(mscan::dispatch_conv_fwd(p, dt == MAMBA_F32 ? 0 : 1, vec,
                                             static_cast<hipStream_t>(stream)));
}

mamba_status mamba_conv1d_silu_bwd(const void* x, const float* w, const float* b,
                                   const uint8_t* reset, const float* du, int64_t width,
                                   mamba_dtype dt, int64_t batch, int64_t dim, int64_t seqlen,
                                   float* dx, float* dw, float* db, void* stream) {
  mamba_status st = check_sizes(dt, MAMBA_DISC_ZOH, batch, dim, 1, seqlen);
  if (st != MAMBA_OK) return st;
  if (width < 1 || width > 4) return MAMBA_ERR_UNSUPPORTED;
  if (!x || !w || !du || !dx || !dw) return MAMBA_ERR_NULL_PTR;
  if ((b == nullptr) != (db == nullptr)) return MAMBA_ERR_INVALID;
  const void* ptrs[] = {x, w, b, du, dx, dw, db};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_ALIGNMENT;
  mscan::ConvParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.w = w; p.b = b; p.reset = reset; p.du = du; p.dx = dx; p.dw = dw; p.db = db;
  p.batch = batch; p.dim = dim; p.L = seqlen; p.nchannels = batch * dim;
  p.tiles = mscan::conv_tiles(seqlen); p.W = (int)width;
  if (p.nchannels * p.tiles > (int64_t)0x7FFFFFFF) return MAMBA_ERR_UNSUPPORTED;
  // vector loads need 16-byte rows for both x and the float32 du / dx
  const bool vec = rows_aligned16(seqlen, elem_size(dt)) && rows_aligned16(seqlen, 4);
  return hip_status(mscan::dispatch_conv_bwd(p, dt == MAMBA_F32 ? 0 : 1, vec,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"

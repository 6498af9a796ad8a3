// Kernel parameter blocks and launcher declarations shared by the C-ABI layer
// (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

// Items (time steps) each lane owns per chunk: forward and backward.
constexpr int kItems = 8;
constexpr int kItemsBwd = 8;
// Threads per workgroup of the scan kernels (4 waves of 64).
constexpr int kBlock = 256;

struct FwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;          // nullable
  const void* z;           // nullable
  const float* bias;       // nullable
  const float* h0;         // nullable
  void* out;
  float* last_state;       // nullable
  float* chunk_states;     // (nchannels, nchunks, N) state at each 128-step chunk start: written
                           // by the recompute mode, and by the output mode when non-null
  int64_t batch, dim, L;
  int64_t nchannels;       // batch * dim
  int64_t groups;          // channel groups per batch row (one block each)
  // Sequence segments (long sequences with few channels): each block covers
  // seg_chunks chunks of one channel group.  seg_chunks = 0, nseg = 1: the
  // whole sequence.
  int64_t seg_chunks;
  int64_t nseg;
  float* seg_h0;           // (nchannels, nseg, N): state entering each segment (carry kernel)
  float* seg_state;        // local pass: (nchannels, nseg, N) end state from a zero start
  float* seg_dsum;         // local pass: (nchannels, nseg) sum of delta over the segment
  float* seg_keep;         // local pass: (nchannels, nseg) 0 if the segment has a reset, else 1
  const uint8_t* reset;    // nullable (batch, L): zero the state before each flagged step
  int seg_pass;            // SegPass
  int N;
  int softplus;
};

// What a forward-kernel launch computes.
enum FwdMode : int {
  kModeOut = 0,           // outputs (and the last state)
  kModeChunkStates = 1,   // only the state at every chunk start (backward recompute)
  kModeSegSummary = 2,    // only each segment's end state from zero and its delta sum
};

// Which pass of a (possibly segmented) run a forward-kernel launch is.
enum SegPass : int {
  kSegWhole = 0,          // from h0, or from p.seg_h0 per segment when that is set
  kSegLocal = 1,          // every segment from a zero state; writes the segment summaries
  kSegFix = 2,            // each segment's first chunks again from its entering state
};

struct BwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;          // nullable
  const void* z;           // nullable
  const float* bias;       // nullable
  const float* h0;         // nullable
  const void* dout;
  float* du;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;               // nullable
  float* dz;               // nullable
  float* dbias;            // nullable
  float* dh0;              // nullable
  const float* chunk_states;  // workspace: (nchannels, nchunks, N) states at chunk starts
  int* deferred;           // workspace: one flag per block (blocks with A ~ 0, ZOH)
  const uint8_t* reset;    // nullable (batch, L): zero the state before each flagged step
  int64_t batch, dim, L;
  int64_t nchannels;
  int64_t nchunks;         // chunks of 16*kItemsBwd steps
  int64_t groups;          // channel groups per batch row (ceil(dim / channels per block))
  // Sequence segments, as in FwdParams: each block walks seg_chunks chunks of
  // one channel group (seg_chunks = 0, nseg = 1: the whole sequence).
  int64_t seg_chunks;
  int64_t nseg;
  // adjoint g entering each segment from the later ones, (nchannels, nseg, N)
  // (nullable: zero); written by the carry kernel from the summaries
  float* seg_gin;
  float* seg_gloc;         // summary: (nchannels, nseg, N) adjoint at the segment start, zero g
                           // entering its end
  float* seg_gdsum;        // summary: (nchannels, nseg) sum of delta over the segment
  float* seg_gkeep;        // summary: (nchannels, nseg) 0 if the segment has a reset, else 1
  int N;
  int softplus;
};

struct StepParams {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  int64_t batch, dim;
  int64_t nchannels;
  int N;
  int softplus;
};

// Complex-valued forward (scan_fwd_complex.hip); complex arrays are
// interleaved (re, im) pairs.
struct CplxParams {
  const void* u;
  const void* delta;
  const float2* A;         // (dim, N)
  const float2* B;         // (batch, N, L)
  const float2* C;         // (batch, N, L)
  const float* D;          // nullable
  const void* z;           // nullable
  const float* bias;       // nullable
  const float2* h0;        // nullable (batch, dim, N)
  void* out;
  float2* last_state;      // nullable (batch, dim, N)
  int64_t batch, dim, L;
  int64_t nchannels;
  int64_t groups;          // channel groups of 16 per batch row
  float2* chunk_states;    // (nchannels, nchunks, N) state entering each chunk: the recompute
                           // pass, or checkpoints of the output pass (nullable there)
  // Sequence segments, as in FwdParams (seg_chunks = 0, nseg = 1: the whole
  // sequence).  The summary pass writes each segment's end state from zero
  // and its decay prod(Abar) per state; the carry turns them into the state
  // entering each segment, from which the output and state passes start.
  int64_t seg_chunks;
  int64_t nseg;
  float2* seg_h0;          // (nchannels, nseg, N) state entering each segment (nullable)
  float2* seg_state;       // summary: (nchannels, nseg, N) end state from a zero start
  float2* seg_dec;         // summary: (nchannels, nseg, N) product of Abar over the segment
  const uint8_t* reset;    // nullable (batch, L): zero the state before each flagged step
  int N;                   // <= 16
  int softplus;
};
hipError_t dispatch_scan_fwd_complex(const CplxParams& p, int dtype, int disc, bool vec,
                                     hipStream_t s);
hipError_t dispatch_chunk_states_complex(const CplxParams& p, int dtype, int disc, bool vec,
                                         hipStream_t s);
hipError_t dispatch_seg_summary_complex(const CplxParams& p, int dtype, int disc, bool vec,
                                        hipStream_t s);
// Also writes p.last_state (the state after the last segment) when set.
hipError_t dispatch_seg_carry_complex(const CplxParams& p, hipStream_t s);

// Complex-valued decode step (state_update_complex.hip): one recurrence step
// on a complex state, in place.  B, C are (batch, N) complex, A (dim, N).
struct CplxStepParams {
  float2* state;           // (batch, dim, N)
  const void* u;
  const void* delta;
  const float2* A;
  const float2* B;
  const float2* C;
  const float* D;          // nullable
  const void* z;           // nullable
  const float* bias;       // nullable
  void* out;
  int64_t batch, dim;
  int64_t nchannels;
  int N;                   // <= 16
  int softplus;
};
hipError_t dispatch_state_update_complex(const CplxStepParams& p, int dtype, int disc,
                                         hipStream_t s);

// Complex-valued backward (scan_bwd_complex.hip).
struct CplxBwdParams {
  const void* u;
  const void* delta;
  const float2* A;
  const float2* B;
  const float2* C;
  const float* D;          // nullable
  const void* z;           // nullable
  const float* bias;       // nullable
  const float2* h0;        // nullable
  const void* dout;
  float* du;
  float* ddelta;
  float2* dA;
  float2* dB;
  float2* dC;
  float* dD;               // nullable
  float* dz;               // nullable
  float* dbias;            // nullable
  float2* dh0;             // nullable
  const float2* chunk_states;  // (nchannels, nchunks, N) state entering each 128-step chunk
  int64_t batch, dim, L;
  int64_t nchannels;
  int64_t nchunks;
  int64_t groups;
  // Sequence segments: blocks (batch row, segment, group).  The adjoint
  // entering each segment from the later ones comes from the adjoint summary
  // (G at the segment start from a zero end, and prod(Abar) over the
  // segment) and the reverse carry g <- G + conj(prod Abar) g.
  int64_t seg_chunks;
  int64_t nseg;
  float2* seg_gin;         // (nchannels, nseg, N) adjoint entering each segment (nullable: 0)
  float2* seg_gloc;        // summary: (nchannels, nseg, N)
  float2* seg_gdec;        // summary: (nchannels, nseg, N)
  const uint8_t* reset;    // nullable (batch, L): zero the state before each flagged step
  int N;                   // <= 16
  int softplus;
};
hipError_t dispatch_scan_bwd_complex(const CplxBwdParams& p, int dtype, int disc, bool vec,
                                     hipStream_t s);
hipError_t dispatch_bwd_seg_summary_complex(const CplxBwdParams& p, int dtype, bool vec,
                                            hipStream_t s);
hipError_t dispatch_bwd_seg_carry_complex(const CplxBwdParams& p, hipStream_t s);

// Short causal convolution + SiLU (conv1d_silu.hip).
struct ConvParams {
  const void* x;           // (batch, dim, L), sequence dtype
  const float* w;          // (dim, W)
  const float* b;          // (dim), nullable
  const uint8_t* reset;    // (batch, L), nullable
  void* u;                 // forward output (batch, dim, L), sequence dtype
  const float* du;         // backward input (batch, dim, L)
  float* dx;               // backward outputs
  float* dw;
  float* db;               // nullable (iff b is)
  int64_t batch, dim, L;
  int64_t nchannels;
  int64_t tiles;           // blocks per channel (conv_tiles(L))
  int W;                   // taps, 1..4
};
// The convolution kernels give each thread kConvRun consecutive steps and
// each 256-thread block kConvTile steps of one channel.
constexpr int kConvRun = 8;
constexpr int kConvTile = kConvRun * 256;
inline int64_t conv_tiles(int64_t L) { return (L + kConvTile - 1) / kConvTile; }
hipError_t dispatch_conv_fwd(const ConvParams& p, int dtype, bool vec, hipStream_t s);
hipError_t dispatch_conv_bwd(const ConvParams& p, int dtype, bool vec, hipStream_t s);

// Channels a block of kBlock threads serves when each channel owns `lanes`
// lanes, and the number of such groups per batch row.
inline int channels_per_block(int lanes) { return (kBlock / 64) * (64 / lanes); }
inline int64_t channel_groups(int64_t dim, int lanes) {
  const int64_t cpb = channels_per_block(lanes);
  return (dim + cpb - 1) / cpb;
}

// dtype: 0 = f32, 1 = bf16.  disc: 0 = ZOH, 1 = Euler.  lanes: 16/32/64.
hipError_t dispatch_scan_fwd_f32(const FwdParams& p, int disc, int lanes, bool vec, hipStream_t s);
hipError_t dispatch_scan_fwd_bf16(const FwdParams& p, int disc, int lanes, bool vec, hipStream_t s);
hipError_t dispatch_chunk_states_f32(const FwdParams& p, int disc, int lanes, bool vec,
                                     hipStream_t s);
hipError_t dispatch_chunk_states_bf16(const FwdParams& p, int disc, int lanes, bool vec,
                                      hipStream_t s);
// Packed sequences with reset flags (p.reset != NULL): 16 lanes per channel.
hipError_t dispatch_scan_fwd_reset_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_scan_fwd_reset_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_chunk_states_reset_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_chunk_states_reset_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
// Segmented runs (16 lanes per channel): the summary pass (short segments),
// the carry over segments (also the last state), and the correcting launch of
// the output or chunk-state kernel (long segments), from each segment's
// entering state over the chunks it still changes.
hipError_t dispatch_seg_summary_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_seg_summary_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_seg_summary_reset_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_seg_summary_reset_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
inline hipError_t dispatch_seg_summary(const FwdParams& p, int dtype, int disc, bool vec,
                                       hipStream_t s) {
  if (p.reset)
    return dtype == 0 ? dispatch_seg_summary_reset_f32(p, disc, vec, s)
                      : dispatch_seg_summary_reset_bf16(p, disc, vec, s);
  return dtype == 0 ? dispatch_seg_summary_f32(p, disc, vec, s)
                    : dispatch_seg_summary_bf16(p, disc, vec, s);
}
hipError_t dispatch_seg_carry(const FwdParams& p, hipStream_t s);
hipError_t dispatch_scan_fwd_fix_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_scan_fwd_fix_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_scan_fwd_fix_reset_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_scan_fwd_fix_reset_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_chunk_states_fix_f32(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_chunk_states_fix_bf16(const FwdParams& p, int disc, bool vec, hipStream_t s);
hipError_t dispatch_chunk_states_fix_reset_f32(const FwdParams& p, int disc, bool vec,
                                               hipStream_t s);
hipError_t dispatch_chunk_states_fix_reset_bf16(const FwdParams& p, int disc, bool vec,
                                                hipStream_t s);
inline hipError_t dispatch_scan_fwd_fix(const FwdParams& p, int dtype, int disc, bool vec,
                                        hipStream_t s) {
  if (p.reset)
    return dtype == 0 ? dispatch_scan_fwd_fix_reset_f32(p, disc, vec, s)
                      : dispatch_scan_fwd_fix_reset_bf16(p, disc, vec, s);
  return dtype == 0 ? dispatch_scan_fwd_fix_f32(p, disc, vec, s)
                    : dispatch_scan_fwd_fix_bf16(p, disc, vec, s);
}
inline hipError_t dispatch_chunk_states_fix(const FwdParams& p, int dtype, int disc, bool vec,
                                            hipStream_t s) {
  if (p.reset)
    return dtype == 0 ? dispatch_chunk_states_fix_reset_f32(p, disc, vec, s)
                      : dispatch_chunk_states_fix_reset_bf16(p, disc, vec, s);
  return dtype == 0 ? dispatch_chunk_states_fix_f32(p, disc, vec, s)
                    : dispatch_chunk_states_fix_bf16(p, disc, vec, s);
}
inline hipError_t dispatch_scan_fwd(const FwdParams& p, int dtype, int disc, int lanes, bool vec,
                                    hipStream_t s) {
  if (p.reset)
    return dtype == 0 ? dispatch_scan_fwd_reset_f32(p, disc, vec, s)
                      : dispatch_scan_fwd_reset_bf16(p, disc, vec, s);
  return dtype == 0 ? dispatch_scan_fwd_f32(p, disc, lanes, vec, s)
                    : dispatch_scan_fwd_bf16(p, disc, lanes, vec, s);
}
// Backward: chunk-state recompute, reverse adjoint scan, then reductions.
inline hipError_t dispatch_chunk_states(const FwdParams& p, int dtype, int disc, int lanes,
                                        bool vec, hipStream_t s) {
  if (p.reset)
    return dtype == 0 ? dispatch_chunk_states_reset_f32(p, disc, vec, s)
                      : dispatch_chunk_states_reset_bf16(p, disc, vec, s);
  return dtype == 0 ? dispatch_chunk_states_f32(p, disc, lanes, vec, s)
                    : dispatch_chunk_states_bf16(p, disc, lanes, vec, s);
}
// The backward always spreads a channel over 16 lanes (kBwdLanes).
constexpr int kBwdLanes = 16;
// Without reset flags, with N <= 16 and in one pass (no sequence segments)
// the backward takes 12-wave blocks (48 channels, one per CU) when they number
// at least this many, else 4-wave blocks (16 channels, three per CU).  From
// 171 wide blocks on, the narrow ones would put a third block on some CU, so
// both take a full CU's turn and the wide blocks' fewer atomics win; below,
// the narrow ones finish in two thirds of that.  Segmented runs (many short
// blocks per channel group) measured faster with narrow blocks.
constexpr int64_t kBwdWideMinBlocks = 171;
// Backward launchers, one per (dtype, reset flags, state-size variant):
// NT = 16 for N <= 16, NT = 64 for N <= 64.  ev_begin / ev_end (nullable) are
// recorded on the stream right before and after the main backward kernel,
// for timing it alone.
#define MSCAN_BWD_DECL(NAME)                                                             \
  hipError_t NAME(const BwdParams& p, int disc, bool vec, hipStream_t s, hipEvent_t ev_begin, \
                  hipEvent_t ev_end);
MSCAN_BWD_DECL(dispatch_scan_bwd_f32_n16)
MSCAN_BWD_DECL(dispatch_scan_bwd_f32_n64)
MSCAN_BWD_DECL(dispatch_scan_bwd_bf16_n16)
MSCAN_BWD_DECL(dispatch_scan_bwd_bf16_n64)
MSCAN_BWD_DECL(dispatch_scan_bwd_reset_f32_n16)
MSCAN_BWD_DECL(dispatch_scan_bwd_reset_f32_n64)
MSCAN_BWD_DECL(dispatch_scan_bwd_reset_bf16_n16)
MSCAN_BWD_DECL(dispatch_scan_bwd_reset_bf16_n64)
#undef MSCAN_BWD_DECL
inline hipError_t dispatch_scan_bwd(const BwdParams& p, int dtype, int disc, bool vec,
                                    hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const bool small = p.N <= 16;
  if (p.reset) {
    if (dtype == 0)
      return small ? dispatch_scan_bwd_reset_f32_n16(p, disc, vec, s, ev_begin, ev_end)
                   : dispatch_scan_bwd_reset_f32_n64(p, disc, vec, s, ev_begin, ev_end);
    return small ? dispatch_scan_bwd_reset_bf16_n16(p, disc, vec, s, ev_begin, ev_end)
                 : dispatch_scan_bwd_reset_bf16_n64(p, disc, vec, s, ev_begin, ev_end);
  }
  if (dtype == 0)
    return small ? dispatch_scan_bwd_f32_n16(p, disc, vec, s, ev_begin, ev_end)
                 : dispatch_scan_bwd_f32_n64(p, disc, vec, s, ev_begin, ev_end);
  return small ? dispatch_scan_bwd_bf16_n16(p, disc, vec, s, ev_begin, ev_end)
               : dispatch_scan_bwd_bf16_n64(p, disc, vec, s, ev_begin, ev_end);
}
// Segmented backward, adjoint side (scan_bwd_seg.hip): each segment's adjoint
// at its start from a zero adjoint at its end, then the carry over segments
// in reverse order into p.seg_gin.
hipError_t dispatch_bwd_seg_summary(const BwdParams& p, int dtype, bool vec, hipStream_t s);
hipError_t dispatch_bwd_seg_carry(const BwdParams& p, hipStream_t s);
hipError_t dispatch_state_update(const StepParams& p, int dtype, int disc, hipStream_t stream);

}  // namespace mscan

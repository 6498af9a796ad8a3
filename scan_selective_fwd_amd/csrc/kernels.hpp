// Kernel parameter blocks and launcher declarations shared by the C-ABI layer
// (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

// Items (time steps) each lane owns per chunk: forward and backward.
constexpr int kItems = 16;
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
  float* chunk_states;     // states-only mode: (nchannels, nchunks, N) state at each chunk start
  int64_t batch, dim, L;
  int64_t nchannels;       // batch * dim
  int N;
  int softplus;
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
  float* part_bc;          // workspace: (batch, groups, 2, N, L) partial dB / dC per channel group
  float* part_a;           // workspace: (batch, dim, N) partial dA per batch row
  float* part_d;           // workspace: (batch, dim, 2) partial dD, ddelta_bias per batch row
  int64_t batch, dim, L;
  int64_t nchannels;
  int64_t nchunks;         // chunks of R*kItemsBwd steps
  int64_t groups;          // channel groups per batch row (ceil(dim / channels per block))
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

// dtype: 0 = f32, 1 = bf16.  disc: 0 = ZOH, 1 = Euler.  lanes: 16/32/64.
hipError_t dispatch_scan_fwd(const FwdParams& p, int dtype, int disc, int lanes, bool vec,
                             hipStream_t stream);
// Backward: chunk-state recompute, reverse adjoint scan, then reductions.
hipError_t dispatch_chunk_states(const FwdParams& p, int dtype, int disc, int lanes, bool vec,
                                 hipStream_t stream);
hipError_t dispatch_scan_bwd(const BwdParams& p, int dtype, int disc, int lanes, bool vec,
                             hipStream_t stream);
hipError_t launch_bwd_reduce(const BwdParams& p, hipStream_t stream);
int64_t bwd_groups(int64_t dim, int lanes);
hipError_t dispatch_state_update(const StepParams& p, int dtype, int disc, hipStream_t stream);

}  // namespace mscan

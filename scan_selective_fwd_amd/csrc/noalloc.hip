// The allocation-free backward entry point (mamba_scan_bwd_noalloc): the
// buffers mamba_scan_bwd takes from its workspace argument live in a
// file-scope device array instead.
//
// The array is a __device__ variable of this code object, so every GPU the
// library is loaded on holds its own copy for the life of the process; its
// device address is looked up per GPU (hipGetSymbolAddress, with that GPU
// current) on the first call made there and kept.  In host code the array's
// name is only a host-side stand-in: the kernels receive the looked-up
// address, never the name.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mamba_scan.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MAMBA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch` per GPU, once looked up
std::mutex g_scratch_mu;

// The current GPU's copy of the array (looked up on first use there).
mamba_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MAMBA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MAMBA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MAMBA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MAMBA_OK;
}

}  // namespace

extern "C" mamba_status mamba_scan_bwd_noalloc(
    const void* u, const void* delta, const float* A, const void* B, const void* C,
    const float* D, const void* z, const float* delta_bias, const float* h0, const void* dout,
    int delta_softplus, mamba_disc disc, mamba_dtype dt, int64_t batch, int64_t dim,
    int64_t dstate, int64_t seqlen, float* du, float* ddelta, float* dA, float* dB, float* dC,
    float* dD, float* dz, float* ddelta_bias, float* dh0, void* stream) {
  // size limit first: a problem that cannot fit is refused before any device
  // call; the automatic choice may still run in one pass when its segmented
  // layout does not fit (mamba_scan_bwd falls back by itself)
  const size_t one_pass =
      mamba_scan_bwd_workspace_size_ex(batch, dim, dstate, seqlen, dt, 0, 1);
  if (one_pass == SIZE_MAX) {
    // invalid sizes: let the full argument checks name the error
    return mamba_scan_bwd(u, delta, A, B, C, D, z, delta_bias, h0, dout, delta_softplus, disc,
                          dt, batch, dim, dstate, seqlen, du, ddelta, dA, dB, dC, dD, dz,
                          ddelta_bias, dh0, nullptr, 0, stream);
  }
  if (one_pass > MAMBA_NOALLOC_SCRATCH_BYTES) return MAMBA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const mamba_status st = current_scratch(&ws);
  if (st != MAMBA_OK) return st;
  return mamba_scan_bwd(u, delta, A, B, C, D, z, delta_bias, h0, dout, delta_softplus, disc, dt,
                        batch, dim, dstate, seqlen, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                        dh0, ws, MAMBA_NOALLOC_SCRATCH_BYTES, stream);
}

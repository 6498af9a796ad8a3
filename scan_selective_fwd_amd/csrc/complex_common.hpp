// Complex float32 arithmetic on (re, im) float2 pairs and the complex affine
// scan step shared by the complex-valued forward and backward kernels.
#pragma once

#include "device_common.hpp"

namespace mscan {

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(__builtin_fmaf(a.x, b.x, -a.y * b.y), __builtin_fmaf(a.x, b.y, a.y * b.x));
}
// a * b + c
__device__ __forceinline__ float2 cfma(float2 a, float2 b, float2 c) {
  return make_float2(__builtin_fmaf(a.x, b.x, __builtin_fmaf(-a.y, b.y, c.x)),
                     __builtin_fmaf(a.x, b.y, __builtin_fmaf(a.y, b.x, c.y)));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// Re(conj(a) * b)
__device__ __forceinline__ float cdot(float2 a, float2 b) {
  return __builtin_fmaf(a.x, b.x, a.y * b.y);
}

// One step of a scan of complex affine pairs (A, B) over lanes: combine with
// the pair the DPP pattern CTRL brings from another lane (row_shr: the
// earlier lane, prefix; row_shl: the later lane, suffix).  A lane without a
// source lane keeps its pair (the identity (1, 0) enters).
template <int CTRL>
__device__ __forceinline__ void cplx_scan_step(float2& A, float2& Bv) {
  const float2 Ap = make_float2(dpp_mov<CTRL>(1.0f, A.x), dpp_mov<CTRL>(0.0f, A.y));
  const float2 Bp = make_float2(dpp_mov<CTRL>(0.0f, Bv.x), dpp_mov<CTRL>(0.0f, Bv.y));
  Bv = cfma(A, Bp, Bv);
  A = cmul(A, Ap);
}

}  // namespace mscan

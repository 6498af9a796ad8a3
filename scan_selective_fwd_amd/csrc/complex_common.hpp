// Complex float32 arithmetic on (re, im) float2 pairs and the complex affine
// scans shared by the complex-valued forward and backward kernels.
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

// exp(dt * a) for a = ar + i ai given as ar2 = ar * log2(e) and air =
// ai / (2 pi): the hardware exponential and sine / cosine (which take
// revolutions), without the scaling multiplies of the generic forms.
__device__ __forceinline__ float2 cexp_scaled(float dt, float ar2, float air) {
  const float mag = fast_exp2(dt * ar2);
  const float rev = dt * air;
  return make_float2(mag * __builtin_amdgcn_cosf(rev), mag * __builtin_amdgcn_sinf(rev));
}

// exp(dt * a) as cexp_scaled, and also exp(dt * a) - 1 without cancellation
// (the ZOH coefficient (Abar - 1)/A of a complex A; chapterpal.com page,
// Knowl 1, step 3).  With x = dt a = xr + i xi:
//   Abar - 1 = (expm1(xr) cos(xi) + (cos(xi) - 1)) + i e^xr sin(xi).
// The imaginary part has no cancellation (v_sin_f32 is relative-accurate
// near 0: within 9e-7, measured on gfx950).  expm1(xr) is expm1_zoh; cos(xi)
// - 1 is the larger of two lower bounds, its alternating Taylor series cut
// after the y^6 term (-y^2/2 + y^4/24 - y^6/720 <= cos y - 1 for every real
// y) and the hardware cosine minus 1 + 2^-22 (v_cos_f32 measured within
// 1.3e-7 near 1), so its relative error stays below about 3e-6.
constexpr float kCos2 = 19.739208802178716f;    // (2 pi)^2 / 2
constexpr float kCos4 = 64.939394022668291f;    // (2 pi)^4 / 24
constexpr float kCos6 = 85.456817206693722f;    // (2 pi)^6 / 720
constexpr float kCosBound = 1.00000023841857910f;   // 1 + 2^-22
__device__ __forceinline__ float2 cexp_expm1_scaled(float dt, float ar2, float air, float2& em1) {
  const float zr = dt * ar2;
  const float mag = fast_exp2(zr);
  const float rev = dt * air;            // xi in revolutions
  const float co = __builtin_amdgcn_cosf(rev), si = __builtin_amdgcn_sinf(rev);
  const float w = rev * rev;
  const float cm1 = __builtin_fmaxf(w * __builtin_fmaf(w, __builtin_fmaf(w, -kCos6, kCos4), -kCos2),
                                    co - kCosBound);
  em1 = make_float2(__builtin_fmaf(expm1_zoh(zr, mag), co, cm1), mag * si);
  return make_float2(mag * co, mag * si);
}

// d/dA of the ZOH coefficient (e^x - 1)/A of a complex A at fixed dt:
// dt^2 psi(x), psi(x) = (x e^x - e^x + 1)/x^2 = 1/2 + x/3 + x^2/8 + x^3/30 +
// ... with x = dt a.  Below |x| = 0.17 the series (its first omitted term,
// x^4/144, is at most 1.2e-5 of psi there).  Above, (dt Abar - coef)/A,
// from the exact identity A d(coef)/dA = dt Abar - coef, with coef = (Abar -
// 1)/A the accurate coefficient the replay formed: the difference cancels
// only to O(|x|) of its terms, so coef's and Abar's errors grow by at most
// about 2/|x| (12 at the threshold), where the closed form (Abar (x - 1) +
// 1)/A^2 divides Abar's absolute error by |x|^2 / 2.  Worst relative error
// about 1.5e-5 (float32 emulation with the hardware exp, sin and cos off by
// their measured errors).  At A = 0 (ia = 0, coef = dt) the series is taken.
__device__ __forceinline__ float2 cdcoef_dA(float dt, float2 a, float2 ab, float2 coef, float2 ia) {
  const float2 x = cscale(a, dt);
  float2 w = make_float2(__builtin_fmaf(x.x, 1.0f / 30.0f, 0.125f), x.y * (1.0f / 30.0f));
  w = cmul(x, w);
  w.x += 1.0f / 3.0f;
  w = cmul(x, w);
  w.x += 0.5f;
  const float2 series = cscale(w, dt * dt);
  const float2 closed =
      cmul(make_float2(__builtin_fmaf(dt, ab.x, -coef.x), __builtin_fmaf(dt, ab.y, -coef.y)), ia);
  const bool small = __builtin_fmaf(x.x, x.x, x.y * x.y) < 0.0289f;   // |x| < 0.17
  return small ? series : closed;
}

// (ab - 1) q, with q = (1/A) B u computed once per step: the ZOH term
// Bbar u = (Abar - 1)/A B u.
__device__ __forceinline__ float2 cmul_minus_one(float2 ab, float2 q) {
  return make_float2(__builtin_fmaf(ab.x, q.x, __builtin_fmaf(-ab.y, q.y, -q.x)),
                     __builtin_fmaf(ab.x, q.y, __builtin_fmaf(ab.y, q.x, -q.y)));
}

// Scans of complex affine pairs (A, B) over the 16 lanes of a row, combining
// each lane with the pair of the lane the DPP pattern names (row_shr: the
// earlier lane, prefix; row_shl: the later lane, suffix), in four steps
// (shift 1, 2, 4, 8) of DPP-modified VOP2 instructions.  Per step, with (a, b) this lane's pair and
// (a', b') the source lane's:  b <- a b' + b  and  a <- a a'.  A lane whose
// source lies outside its row is not written by the DPP instructions: t0 then
// keeps 0 and the new a starts from the lane's own a, so the lane keeps its
// pair (the identity enters).  12 instructions per step (moving each operand
// with the update_dpp builtin takes 16); two wait states precede each step's
// first DPP read.
#define MSCAN_CPLX_DPP_STEP(CTRL)                                               \
  "s_nop 1\n\t"                                                                 \
  "v_mov_b32 %2, 0\n\t"                                                         \
  "v_mov_b32_dpp %2, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %1, %0, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
  "v_fmac_f32 %1, %2, %5\n\t"                                                   \
  "v_fmac_f32_dpp %0, %0, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
  "v_fma_f32 %0, -%2, %6, %0\n\t"                                               \
  "v_mov_b32 %3, %5\n\t"                                                        \
  "v_mul_f32_dpp %3, %5, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
  "v_fmac_f32_dpp %3, %6, -%6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
  "v_mov_b32 %4, %6\n\t"                                                        \
  "v_mul_f32_dpp %4, %5, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
  "v_fmac_f32_dpp %4, %6, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"

#define MSCAN_CPLX_DPP_STEP_CALL(CTRL)                                               \
  do {                                                                                \
    float t0, nx, ny;                                                                 \
    asm volatile(MSCAN_CPLX_DPP_STEP(CTRL)                                            \
                 : "+v"(B.x), "+v"(B.y), "=&v"(t0), "=&v"(nx), "=&v"(ny)             \
                 : "v"(A.x), "v"(A.y));                                               \
    A = make_float2(nx, ny);                                                          \
  } while (0)

// Inclusive prefix scan over each 16-lane row (row_shr: the earlier lane).
__device__ __forceinline__ void cplx_scan_prefix_row(float2& A, float2& B) {
  MSCAN_CPLX_DPP_STEP_CALL("row_shr:1");
  MSCAN_CPLX_DPP_STEP_CALL("row_shr:2");
  MSCAN_CPLX_DPP_STEP_CALL("row_shr:4");
  MSCAN_CPLX_DPP_STEP_CALL("row_shr:8");
}

// Inclusive suffix scan over each 16-lane row (row_shl: the later lane).
__device__ __forceinline__ void cplx_scan_suffix_row(float2& A, float2& B) {
  MSCAN_CPLX_DPP_STEP_CALL("row_shl:1");
  MSCAN_CPLX_DPP_STEP_CALL("row_shl:2");
  MSCAN_CPLX_DPP_STEP_CALL("row_shl:4");
  MSCAN_CPLX_DPP_STEP_CALL("row_shl:8");
}

#undef MSCAN_CPLX_DPP_STEP_CALL
#undef MSCAN_CPLX_DPP_STEP

}  // namespace mscan

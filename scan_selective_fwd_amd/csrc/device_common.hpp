// Device helpers shared by the selective-scan kernels (gfx950 / CDNA4, wave64).
//
// Lane layout used by the scan kernels: a channel (one (b, d) pair) owns R
// consecutive lanes of a wave (R = 16, 32 or 64), each lane owning K
// consecutive time steps of the current chunk, so a chunk covers R*K steps.
// The recurrence h_t = a_t h_{t-1} + b_t composes affine maps h -> a h + b;
// composition is associative ((a1,b1) then (a2,b2) = (a2 a1, a2 b1 + b2)),
// which is what lets the scan run as a tree across lanes (paper-graph-ui
// summary of the Mamba paper, section 3.4, "The parallel scan"; trishampatil
// essay, Part III §2).  The cross-lane steps use DPP row shifts/broadcasts,
// which move data between lanes inside the VALU without touching LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

typedef uint16_t bf16_t;  // bfloat16 stored as its 16-bit pattern

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInv2Pi = 0.15915494309189535f;   // 1 / (2 pi)
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// DPP moves.  With bound_ctrl off, a lane whose source lane is invalid (or
// whose row is masked off) keeps `old`: the scans pass the identity element
// of the operation there.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp_mov(float old, float src) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, src),
                                         CTRL, ROW_MASK, BANK_MASK, false));
}

enum : int {
  kRowShr1 = 0x111,
  kRowShr2 = 0x112,
  kRowShr4 = 0x114,
  kRowShr8 = 0x118,
  kWaveShr1 = 0x138,
  kRowBcast15 = 0x142,
  kRowBcast31 = 0x143,
};

// One step of the inclusive scan: combine with the pair held by the source
// lane of the DPP pattern (the earlier segment).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void affine_step(float& A, float& B) {
  float Ap = dpp_mov<CTRL, ROW_MASK>(1.0f, A);
  float Bp = dpp_mov<CTRL, ROW_MASK>(0.0f, B);
  B = __builtin_fmaf(A, Bp, B);
  A = A * Ap;
}

// Inclusive scan of affine pairs over groups of R lanes (R = 16, 32, 64).
// On return lane i of a group holds the composition of lanes 0..i.
template <int R>
__device__ __forceinline__ void affine_scan_inclusive(float& A, float& B) {
  static_assert(R == 16 || R == 32 || R == 64, "R");
  affine_step<kRowShr1>(A, B);
  affine_step<kRowShr2>(A, B);
  affine_step<kRowShr4>(A, B);
  affine_step<kRowShr8>(A, B);
  if constexpr (R >= 32) affine_step<kRowBcast15, 0xA>(A, B);
  if constexpr (R == 64) affine_step<kRowBcast31, 0xC>(A, B);
}

// The same inclusive scan written with DPP-modified VOP2 instructions: each
// step is one v_fmac_f32_dpp and one v_mul_f32_dpp.  A lane whose DPP source
// is outside its row (or in a row masked off) is not written, which leaves
// it holding its own pair -- the identity of the combine -- without the
// separate identity moves the builtin form needs.  Two wait states separate
// a VALU write from a DPP read of the same register (s_nop 1).  Requires all
// 64 lanes active (it is only used outside divergent code).
template <int R>
__device__ __forceinline__ void affine_scan_inclusive_fused(float& A, float& B) {
  static_assert(R == 16 || R == 32 || R == 64, "R");
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(A), "+v"(B));
  if constexpr (R >= 32)
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        : "+v"(A), "+v"(B));
  if constexpr (R == 64)
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        : "+v"(A), "+v"(B));
}

// Suffix counterpart over 16-lane rows: lane i ends with the composition of
// lanes i..15 of its row, later lanes applied first (row_shl sources).
__device__ __forceinline__ void affine_suffix_scan_row_fused(float& A, float& B) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(A), "+v"(B));
}

// A prefix scan of (A1, B1) (row_shr sources, as affine_scan_inclusive_fused
// with R = 16) and a suffix scan of (A2, B2) (row_shl sources, as
// affine_suffix_scan_row_fused), interleaved.  The two are independent, so
// every DPP read finds its source register written three instructions
// earlier and only the first step needs wait states.  The final products
// A1, A2 of the last step are not formed: the callers use only B1, B2 (on
// return A1, A2 hold the products over the first 8 lanes' spans).
__device__ __forceinline__ void dual_scan_row_fused(float& A1, float& B1, float& A2, float& B2) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %2 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %2, %2 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %2 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %2, %2 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %2 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %2, %2 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %2 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      : "+v"(A1), "+v"(B1), "+v"(A2), "+v"(B2));
}

// Sum over each 16-lane row, result in the row's lane 15 (the other lanes
// hold partial sums): an inclusive DPP add-scan with row_shr sources.
__device__ __forceinline__ float row_sum_to_last(float v) {
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(v));
  return v;
}

// One stage-1 exchange of the row reduce-scatter: for items (x, y) of the
// four 16-lane rows returns, in rows 0 and 2, x summed over the row pair
// (0,1) or (2,3), and in rows 1 and 3 the same for y.
__device__ __forceinline__ float rs_pair16(float x, float y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Stage 2: from two stage-1 results, rows 0/1 get the first summed over all
// four rows, rows 2/3 the second.
__device__ __forceinline__ float rs_pair32(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Compiler-level fence: memory operations are not moved across it.  Used
// between the iterations of unrolled loops so that each iteration's loads
// stay with it instead of being hoisted en masse.
__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }

// Returns v, hidden from the optimizer: what is computed from the result is
// computed again at each use instead of being kept in registers from an
// earlier one.  Used for per-thread addresses in the backward kernels' chunk
// loops: kept, they are spilled, and reloading a spill (an s_waitcnt
// vmcnt(0)) waits for every store, atomic and prefetch load still in flight.
__device__ __forceinline__ int opaque_int(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Reduce-scatter over the 4 rows of a wave: v[k] (K = 8 items) of the four
// 16-lane rows are summed so that lane (row r, j) returns out[m] = sum over
// rows of v[4m + r] at position j (m = 0, 1).  Uses gfx950's
// v_permlane16_swap (odd rows of one register <-> even rows of another) and
// v_permlane32_swap (upper half <-> lower half): 6 swaps and 6 adds.
__device__ __forceinline__ void reduce_scatter_rows8(const float (&v)[8], float (&out)[2]) {
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[2 * i]),
                                              __float_as_uint(v[2 * i + 1]), false, false);
    s[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);   // rows 0,2: item 2i; rows 1,3: 2i+1
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s[2 * m]),
                                              __float_as_uint(s[2 * m + 1]), false, false);
    out[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // row r: item 4m + r
  }
}

// LDS tile of fp32 rows in which lane j of a 16..64-lane group reads its K
// consecutive elements [j*K, j*K+K) as K/4 16-byte granules.  Granule g of a
// row is stored at g ^ ((g >> 4) & (K/4 - 1)): within every 16 consecutive
// lanes the granules a ds_read_b128 touches then cover all 64 banks once.
template <int K>
__device__ __forceinline__ int tile_granule(int g) {
  constexpr int GPL = K / 4;
  return g ^ ((g >> 4) & (GPL - 1));
}

// Carry hand-off between chunks without a broadcast: the state leaving the
// last lane of a channel's group is moved to the group's FIRST lane (the only
// lane that uses it: it is folded into lane 0's summary before the next
// scan).  R = 16: DPP row_ror:1; R = 64: wave_ror:1; R = 32: two readlanes.
template <int R>
__device__ __forceinline__ float last_to_first(float v) {
  if constexpr (R == 16) {
    return dpp_mov<0x121 /*row_ror:1*/>(v, v);
  } else if constexpr (R == 64) {
    return dpp_mov<0x13C /*wave_ror:1*/>(v, v);
  } else {
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    return (__lane_id() & 32) ? hi : lo;
  }
}

// Reverse hand-off for 16-lane rows: lane 0's value moves to lane 15.
__device__ __forceinline__ float row_first_to_last(float v) {
  return dpp_mov<0x12F /*row_ror:15*/>(v, v);
}

// Value of lane R-1 of this lane's group, broadcast to the whole group.
template <int R>
__device__ __forceinline__ float group_last(float v) {
  if constexpr (R == 16) {
    // ds_swizzle bit mode: lane reads ((lane & 0x10) | 0x0F) within 32 lanes.
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F0));
  } else if constexpr (R == 32) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x3E0));
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  }
}

// Value of lane 0 of this lane's group, broadcast to the whole group.
template <int R>
__device__ __forceinline__ float group_first(float v) {
  if constexpr (R == 16) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x010));
  } else if constexpr (R == 32) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x000));
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  }
}

// Lane i receives lane i-1 of its group; lane 0 of the group receives `first`.
template <int R>
__device__ __forceinline__ float group_shift_right(float v, float first) {
  if constexpr (R == 16) {
    return dpp_mov<kRowShr1>(first, v);
  } else {
    float s = dpp_mov<kWaveShr1>(first, v);
    if constexpr (R == 32) s = ((__lane_id() & 31) == 0) ? first : s;
    return s;
  }
}

// Sum over the R lanes of a group, result in every lane of the group.
template <int R>
__device__ __forceinline__ float group_sum(float v) {
  // butterfly with ds_swizzle xor (within 32) and a readlane/permute above.
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                             (0x1F) | (1 << 10)));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                             (0x1F) | (2 << 10)));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                             (0x1F) | (4 << 10)));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                             (0x1F) | (8 << 10)));
  if constexpr (R >= 32)
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                               (0x1F) | (16 << 10)));
  if constexpr (R == 64) v += __shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------------------------------
// Math.  exp and log use the hardware base-2 instructions (v_exp_f32,
// v_log_f32); softplus uses an accurate log1p.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log1p(e) for e in [0, 1]: with w = 1 + e rounded, log1p(e) = log(w) * e /
// (w - 1) when w != 1, and e otherwise.  The quotient e / (w - 1) cancels the
// rounding of w (Goldberg, "What Every Computer Scientist Should Know About
// Floating-Point Arithmetic", 1991, Theorem 4).
__device__ __forceinline__ float log1p_unit(float e) {
  float w = 1.0f + e;
  float den = w - 1.0f;
  float lg = __builtin_amdgcn_logf(w) * kLn2;
  return den == 0.0f ? e : lg * (e * fast_rcp(den));
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}).
__device__ __forceinline__ float softplus(float x) {
  float e = fast_exp(-__builtin_fabsf(x));
  return __builtin_fmaxf(x, 0.0f) + log1p_unit(e);
}

__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + fast_exp(-x)); }
// ---------------------------------------------------------------------------
// The ZOH coefficient without cancellation.  Bbar = (e^x - 1)/A B with
// x = delta A (chapterpal.com page, Knowl 1 "Selective State Space Layer
// (S6)", step 3).  With Abar = e^x rounded, Abar - 1 keeps only the bits of
// Abar below 1: for |x| = 1e-4 the relative error is about 1e-3, and at a
// constant step it does not average out along the recurrence.
//
// expm1 from two lower bounds of e^x - 1:
//   * the cubic Taylor polynomial x + x^2/2 + x^3/6, for every real x (its
//     remainder e^xi x^4/24, Lagrange form, is never negative);
//   * Abar - (1 + 2^-23), for x < ln 2: v_exp_f32 is within 0.78 ulp, at
//     most 9e-8 for results in [0.5, 2) (measured on gfx950 against float64
//     over 16M arguments), below 2^-23.  Above ln 2 Abar's error may exceed
//     2^-23, but it stays below 1e-7 relative to e^x - 1 >= 1 there, where
//     this term is the larger one: the maximum stays accurate.
// Their maximum is within about 5e-6 of e^x - 1 relative: the polynomial
// wins for |x| below about 0.05, the hardware exponential above.  The
// arguments are in exp2 units: z = x log2(e), so x = z ln 2.
// ---------------------------------------------------------------------------
constexpr float kExpm1C2 = 0.24022650695910071f;   // ln(2)^2 / 2
constexpr float kExpm1C3 = 0.05550410866482158f;   // ln(2)^3 / 6
constexpr float kExpBound = 1.00000011920928955f;  // 1 + 2^-23

// e^x - 1 for x = z ln 2, given abar = exp2(z) from the hardware.
__device__ __forceinline__ float expm1_zoh(float z, float abar) {
  const float poly = z * __builtin_fmaf(z, __builtin_fmaf(z, kExpm1C3, kExpm1C2), kLn2);
  return __builtin_fmaxf(poly, abar - kExpBound);
}

// The coefficient itself, (e^x - 1)/A, for A < 0 strictly (the usual case;
// the kernels send blocks with any other A to their general path).  Dividing
// the two lower bounds of expm1_zoh by A < 0 turns them into upper bounds of
// the coefficient, so their minimum is taken:
//   * delta (1 + x/2 + x^2/6), the cubic bound over x = delta A (written in z);
//   * (abar - (1 + 2^-22)) / A, formed as fma(abar, 1/A, -(1 + 2^-22)/A); the
//     bound's margin (2^-22 - 9e-8 relative to 1/A) covers the rounding of the
//     constant -(1 + 2^-22)/A and of the fma.
// Relative error below about 8e-6; one multiply fewer than expm1_zoh(z, abar)
// times 1/A.  mb = -(1 + 2^-22)/A.
constexpr float kCoefC2 = 0.34657359027997264f;    // ln(2) / 2
constexpr float kCoefC3 = 0.08007550231970023f;    // ln(2)^2 / 6
constexpr float kCoefBound = 1.00000023841857910f; // 1 + 2^-22
__device__ __forceinline__ float zoh_coef_neg(float dt, float z, float abar, float ia, float mb) {
  const float poly = dt * __builtin_fmaf(z, __builtin_fmaf(z, kCoefC3, kCoefC2), 1.0f);
  return __builtin_fminf(poly, __builtin_fmaf(abar, ia, mb));
}

// d/dA of the ZOH coefficient (e^x - 1)/A at fixed delta: delta^2 psi(x),
// psi(x) = (x e^x - e^x + 1)/x^2 = 1/2 + x/3 + x^2/8 + x^3/30 + ...  The
// closed form cancels to second order for small x, so below |x| = 0.11 the
// series is used (its first omitted term, x^4/144, is about 2e-6 of psi
// there); above, the closed form is within about 2e-7/x^2 (relative: abar
// carries at most 9e-8 of absolute error, the numerator is about x^2/2).  In the closed form delta^2
// cancels: delta^2 psi = (abar (x - 1) + 1) / A^2, so A = 0 needs no
// special case (the series branch is taken).  dt2 = delta^2, iA2 = 1/A^2.
constexpr float kPsiZ = 0.15869619f;               // 0.11 / ln 2: |x| < 0.11 in z units
constexpr float kPsiC1 = 0.23104906018664844f;     // ln(2) / 3
constexpr float kPsiC2 = 0.06005662673977518f;     // ln(2)^2 / 8
constexpr float kPsiC3 = 0.01110082173296432f;     // ln(2)^3 / 30
__device__ __forceinline__ float dcoef_dA(float z, float abar, float dt2, float iA2) {
  const float series =
      dt2 * __builtin_fmaf(z, __builtin_fmaf(z, __builtin_fmaf(z, kPsiC3, kPsiC2), kPsiC1), 0.5f);
  const float closed = __builtin_fmaf(abar, __builtin_fmaf(z, kLn2, -1.0f), 1.0f) * iA2;
  return __builtin_fabsf(z) < kPsiZ ? series : closed;
}

__device__ __forceinline__ float silu(float x) { return x * sigmoid(x); }

// ---------------------------------------------------------------------------
// Element I/O for float and bfloat16 rows.  `load_k` reads K consecutive
// elements starting at p (16-byte aligned when VEC), `load_k_guarded` reads
// only the first `nvalid` of them (others are 0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (f != f) ? ((u >> 16) | 0x40u) : r;
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  template <int K>
  __device__ __forceinline__ static void load_k(const float* __restrict__ p, float (&v)[K]) {
    static_assert(K % 4 == 0, "K");
#pragma unroll
    for (int i = 0; i < K / 4; ++i) {
      float4 x = reinterpret_cast<const float4*>(p)[i];
      v[4 * i + 0] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  }
  template <int K>
  __device__ __forceinline__ static void load_k_guarded(const float* __restrict__ p, int nvalid,
                                                        float (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = (k < nvalid) ? p[k] : 0.0f;
  }
  template <int K>
  __device__ __forceinline__ static void store_k(float* __restrict__ p, const float (&v)[K]) {
#pragma unroll
    for (int i = 0; i < K / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
  template <int K>
  __device__ __forceinline__ static void store_k_guarded(float* __restrict__ p, int nvalid,
                                                         const float (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k < nvalid) p[k] = v[k];
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

template <>
struct Elem<bf16_t> {
  template <int K>
  __device__ __forceinline__ static void load_k(const bf16_t* __restrict__ p, float (&v)[K]) {
    static_assert(K % 8 == 0, "K");
#pragma unroll
    for (int i = 0; i < K / 8; ++i) {
      uint4 x = reinterpret_cast<const uint4*>(p)[i];
      v[8 * i + 0] = bf16_lo(x.x);
      v[8 * i + 1] = bf16_hi(x.x);
      v[8 * i + 2] = bf16_lo(x.y);
      v[8 * i + 3] = bf16_hi(x.y);
      v[8 * i + 4] = bf16_lo(x.z);
      v[8 * i + 5] = bf16_hi(x.z);
      v[8 * i + 6] = bf16_lo(x.w);
      v[8 * i + 7] = bf16_hi(x.w);
    }
  }
  template <int K>
  __device__ __forceinline__ static void load_k_guarded(const bf16_t* __restrict__ p, int nvalid,
                                                        float (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = (k < nvalid) ? bf16_to_f32(p[k]) : 0.0f;
  }
  template <int K>
  __device__ __forceinline__ static void store_k(bf16_t* __restrict__ p, const float (&v)[K]) {
#pragma unroll
    for (int i = 0; i < K / 8; ++i) {
      uint4 x;
      x.x = f32_to_bf16_bits(v[8 * i + 0]) | (f32_to_bf16_bits(v[8 * i + 1]) << 16);
      x.y = f32_to_bf16_bits(v[8 * i + 2]) | (f32_to_bf16_bits(v[8 * i + 3]) << 16);
      x.z = f32_to_bf16_bits(v[8 * i + 4]) | (f32_to_bf16_bits(v[8 * i + 5]) << 16);
      x.w = f32_to_bf16_bits(v[8 * i + 6]) | (f32_to_bf16_bits(v[8 * i + 7]) << 16);
      reinterpret_cast<uint4*>(p)[i] = x;
    }
  }
  template <int K>
  __device__ __forceinline__ static void store_k_guarded(bf16_t* __restrict__ p, int nvalid,
                                                         const float (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k < nvalid) p[k] = (bf16_t)f32_to_bf16_bits(v[k]);
  }
  __device__ __forceinline__ static float load1(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(bf16_t* p, float v) {
    *p = (bf16_t)f32_to_bf16_bits(v);
  }
};

// Load K elements of a row starting at element offset `t` of a row with
// `L` valid elements; vector loads when the whole run is in range.
template <typename T, int K, bool VEC>
__device__ __forceinline__ void load_run(const T* __restrict__ row, int64_t t, int64_t L,
                                         float (&v)[K]) {
  int64_t rem = L - t;
  int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
  if (VEC && nvalid == K) {
    Elem<T>::template load_k<K>(row + t, v);
  } else {
    Elem<T>::template load_k_guarded<K>(row + t, nvalid, v);
  }
}

template <typename T, int K, bool VEC>
__device__ __forceinline__ void store_run(T* __restrict__ row, int64_t t, int64_t L,
                                          const float (&v)[K]) {
  int64_t rem = L - t;
  int nvalid = rem >= K ? K : (rem < 0 ? 0 : (int)rem);
  if (VEC && nvalid == K) {
    Elem<T>::template store_k<K>(row + t, v);
  } else if (nvalid > 0) {
    Elem<T>::template store_k_guarded<K>(row + t, nvalid, v);
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip (each
// XCD has its own L2).  Remap so that XCD x runs a contiguous range of
// logical blocks; neighbouring channels (which share B and C rows of the same
// batch) then share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  int xcd = bid % kXcd;
  int idx = bid / kXcd;
  int q = nblocks / kXcd, r = nblocks % kXcd;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

}  // namespace mscan

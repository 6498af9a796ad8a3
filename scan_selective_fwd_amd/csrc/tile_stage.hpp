// Cooperative staging of a chunk of the B and C rows into LDS.
//
// All channels of a block belong to one batch row, so they share the B and C
// rows (B, C are (batch, N, L): the pages' selective parameters of shape
// (B, L, N), shared by every channel -- trishampatil essay, Part II §6,
// Algorithm 2).  The block loads each chunk of them from HBM once, with
// coalesced 16-byte loads spread over all its threads, converts to float32,
// and writes an LDS tile that every channel's lanes read from.  The loads for
// chunk c+1 are issued into registers while chunk c is computed; the tile
// for c+1 is written at the end of chunk c into the other LDS buffer.
#pragma once

#include "device_common.hpp"

namespace mscan {

// ROWS rows of TCH elements each; tile row r = which * NT + n (which = 0 for
// B, 1 for C).  Rows with n >= N are neither loaded nor written.
template <typename T, int TCH, int K, int NT, int ROWS, int NTHREADS>
struct TileStager {
  static constexpr int EPG = 16 / (int)sizeof(T);      // elements per 16-byte granule
  static constexpr int GROW = TCH / EPG;               // granules per row
  static constexpr int TOTAL = ROWS * GROW;
  static constexpr int PER_THREAD = (TOTAL + NTHREADS - 1) / NTHREADS;
  static_assert(TCH % EPG == 0, "chunk must hold whole granules");

  uint4 regs[PER_THREAD];

  // Loads the chunk starting at step t0.  `full`: the whole chunk is inside
  // the sequence and rows are 16-byte aligned (vector loads); otherwise each
  // element is loaded alone and steps past L read as 0.
  __device__ __forceinline__ void load(const T* __restrict__ B_b, const T* __restrict__ C_b,
                                       int N, int64_t L, int64_t t0, bool full, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = i * NTHREADS + tid;
      const int row = q / GROW;
      const int col = q - row * GROW;
      const int which = row / NT;
      const int n = row - which * NT;
      regs[i] = make_uint4(0u, 0u, 0u, 0u);
      if (q < TOTAL && n < N) {
        const T* src = (which ? C_b : B_b) + (int64_t)n * L + t0 + (int64_t)col * EPG;
        if (full) {
          regs[i] = *reinterpret_cast<const uint4*>(src);
        } else {
          T tmp[EPG];
#pragma unroll
          for (int e = 0; e < EPG; ++e) {
            const int64_t t = t0 + (int64_t)col * EPG + e;
            tmp[e] = (t < L) ? src[e] : (T)0;
          }
          regs[i] = *reinterpret_cast<const uint4*>(tmp);
        }
      }
    }
  }

  // Writes the loaded chunk to an LDS tile of ROWS x TCH floats.
  __device__ __forceinline__ void store(float* __restrict__ tile, int N, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = i * NTHREADS + tid;
      const int row = q / GROW;
      const int col = q - row * GROW;
      const int n = row - (row / NT) * NT;
      if (q < TOTAL && n < N) {
        float* dst = tile + row * TCH;
        if constexpr (sizeof(T) == 4) {
          const float4 v = make_float4(__uint_as_float(regs[i].x), __uint_as_float(regs[i].y),
                                       __uint_as_float(regs[i].z), __uint_as_float(regs[i].w));
          *reinterpret_cast<float4*>(dst + tile_granule<K>(col) * 4) = v;
        } else {
          const float4 lo = make_float4(bf16_lo(regs[i].x), bf16_hi(regs[i].x),
                                        bf16_lo(regs[i].y), bf16_hi(regs[i].y));
          const float4 hi = make_float4(bf16_lo(regs[i].z), bf16_hi(regs[i].z),
                                        bf16_lo(regs[i].w), bf16_hi(regs[i].w));
          *reinterpret_cast<float4*>(dst + tile_granule<K>(2 * col) * 4) = lo;
          *reinterpret_cast<float4*>(dst + tile_granule<K>(2 * col + 1) * 4) = hi;
        }
      }
    }
  }
};

// Lane j's K consecutive floats [j*K, j*K+K) of one tile row.
template <int K>
__device__ __forceinline__ void tile_read(const float* __restrict__ row, int j, float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K / 4; ++i) {
    const float4 x = *reinterpret_cast<const float4*>(row + tile_granule<K>(j * (K / 4) + i) * 4);
    v[4 * i + 0] = x.x;
    v[4 * i + 1] = x.y;
    v[4 * i + 2] = x.z;
    v[4 * i + 3] = x.w;
  }
}

}  // namespace mscan

// Block summary of one (page, head) bf16 tile: the mean of the page's keys,
// per dim, rounded once (device code shared by the summaries kernel and the
// decode-step kernel, which refreshes the pages that just filled).
//
// One wavefront per tile, 16-byte loads, every row of the tile in flight at
// once. Sums are kept in float64: every bf16 value is
// exact in float64, so the column sum is exact unless its terms span more
// than ~2^41 in magnitude; page_size is a power of two, so the mean is exact
// too, and it is rounded once (nearest-even) to the summary dtype.
#pragma once

#include "ls_internal.h"

namespace ls {

// Tile t = (page_ids[t / num_heads], head t % num_heads); invalid page ids
// are skipped. Rows: page_size (a power of two, at most PMAX); lane l loads
// 16 bytes (8 dims) of rows l / LPR, l / LPR + RPI, ... (LPR = D / 8 lanes
// per row, RPI = 64 / LPR rows per load instruction), every load of the
// tile issued before the first use.
template <int D>
struct SumTile {
  static constexpr int LPR = D / 8;
  static constexpr int RPI = kWave / LPR;
};

template <int D, int PMAX>
__device__ __forceinline__ int sum_tile_load(const uint16_t* __restrict__ keys, int page, int h,
                                             int num_heads, int page_size,
                                             uint4 (&v)[PMAX / SumTile<D>::RPI]) {
  using T = SumTile<D>;
  constexpr int NI = PMAX / T::RPI;
  const int lane = threadIdx.x & 63;
  const int ni = page_size / T::RPI;
  const uint16_t* base = keys + ((size_t)page * num_heads + h) * (size_t)page_size * D +
                         (size_t)(lane / T::LPR) * D + 8 * (lane % T::LPR);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    v[i] = i < ni ? ldg16_stream(base + (size_t)i * T::RPI * D) : make_uint4(0, 0, 0, 0);
  return ni;
}

// The mean of a loaded tile (v, from sum_tile_load) into out[page][h].
template <int D, bool kOutF32, int PMAX>
__device__ __forceinline__ void summary_tile_finish(const uint4 (&v)[PMAX / SumTile<D>::RPI], int ni,
                                                    int page, int h, int num_heads, int page_size,
                                                    void* __restrict__ out) {
  using T = SumTile<D>;
  constexpr int NI = PMAX / T::RPI;
  const int lane = threadIdx.x & 63;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    if (r < ni) {
      const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += (double)bf16_lo(w[j]);
        acc[2 * j + 1] += (double)bf16_hi(w[j]);
      }
    }
  }
  // the RPI row groups' sums of each dim (lanes with the same l % LPR)
#pragma unroll
  for (int off = T::LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += __shfl_xor(acc[j], off, kWave);
  }
  if (lane >= T::LPR) return;
  const double inv = 1.0 / (double)page_size;  // exact: power of two
  const size_t o = ((size_t)page * num_heads + h) * D + 8 * lane;
  if constexpr (kOutF32) {
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = (float)(acc[j] * inv);  // one RNE rounding
    float* dst = reinterpret_cast<float*>(out) + o;
    *reinterpret_cast<float4*>(dst) = make_float4(m[0], m[1], m[2], m[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(m[4], m[5], m[6], m[7]);
  } else {
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pk[j] = (uint32_t)f64_to_bf16_rne(acc[2 * j] * inv) |
              ((uint32_t)f64_to_bf16_rne(acc[2 * j + 1] * inv) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

template <int D, bool kOutF32, int PMAX = 16>
__device__ __forceinline__ void summary_tile_bf16(const uint16_t* __restrict__ keys,
                                                  const int32_t* __restrict__ page_ids, int tile,
                                                  int num_pages, int num_heads, int page_size,
                                                  void* __restrict__ out) {
  const int i = tile / num_heads, h = tile - i * num_heads;
  const int page = page_ids[i];
  if (page < 0 || page >= num_pages) return;
  uint4 v[PMAX / SumTile<D>::RPI];
  const int ni = sum_tile_load<D, PMAX>(keys, page, h, num_heads, page_size, v);
  summary_tile_finish<D, kOutF32, PMAX>(v, ni, page, h, num_heads, page_size, out);
}

// Quest bounds of tile `tile` (as above): the element-wise maximum and
// minimum of the page's keys (Vortex, "Writing an algorithm: vFlow", Quest's
// cache step), stored as out[page][head][0][D] (maximum) and [1][D]
// (minimum). Exact: the maximum and the minimum of bf16 values are bf16
// values, so storing them is a copy of the bits. Keys are taken to be finite
// (a NaN would be skipped by the comparisons).
template <int D, int PMAX = 16>
__device__ __forceinline__ void bounds_tile_bf16(const uint16_t* __restrict__ keys,
                                                 const int32_t* __restrict__ page_ids, int tile,
                                                 int num_pages, int num_heads, int page_size,
                                                 uint16_t* __restrict__ out) {
  using T = SumTile<D>;
  constexpr int NI = PMAX / T::RPI;
  const int lane = threadIdx.x & 63;
  const int i = tile / num_heads, h = tile - i * num_heads;
  const int page = page_ids[i];
  if (page < 0 || page >= num_pages) return;
  uint4 v[NI];
  const int ni = sum_tile_load<D, PMAX>(keys, page, h, num_heads, page_size, v);
  float hi[8], lo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hi[j] = -__builtin_huge_valf();
    lo[j] = __builtin_huge_valf();
  }
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    if (r < ni) {
      const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = bf16_lo(w[j]), a1 = bf16_hi(w[j]);
        hi[2 * j] = fmaxf(hi[2 * j], a0);
        lo[2 * j] = fminf(lo[2 * j], a0);
        hi[2 * j + 1] = fmaxf(hi[2 * j + 1], a1);
        lo[2 * j + 1] = fminf(lo[2 * j + 1], a1);
      }
    }
  }
#pragma unroll
  for (int off = T::LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hi[j] = fmaxf(hi[j], __shfl_xor(hi[j], off, kWave));
      lo[j] = fminf(lo[j], __shfl_xor(lo[j], off, kWave));
    }
  }
  if (lane >= T::LPR) return;
  uint16_t* o = out + ((size_t)page * num_heads + h) * 2 * D + 8 * lane;
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // bf16 values: the top halves are the exact bits
    ph[j] = (__float_as_uint(hi[2 * j]) >> 16) | (__float_as_uint(hi[2 * j + 1]) & 0xffff0000u);
    pl[j] = (__float_as_uint(lo[2 * j]) >> 16) | (__float_as_uint(lo[2 * j + 1]) & 0xffff0000u);
  }
  *reinterpret_cast<uint4*>(o) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
  *reinterpret_cast<uint4*>(o + D) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
}

}  // namespace ls

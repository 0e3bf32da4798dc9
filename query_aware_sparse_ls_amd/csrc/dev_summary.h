// Block summary of one (page, head) bf16 tile: the mean of the page's keys,
// per dim, rounded once (device code shared by the summaries kernel and the
// decode-step kernel, which refreshes the pages that just filled).
//
// One wavefront per tile; lane l owns dims [l*DPL, l*DPL+DPL), so each row
// read is one coalesced access. Sums are kept in float64: every bf16 value is
// exact in float64, so the column sum is exact unless its terms span more
// than ~2^41 in magnitude; page_size is a power of two, so the mean is exact
// too, and it is rounded once (nearest-even) to the summary dtype.
#pragma once

#include "ls_internal.h"

namespace ls {

// Tile t = (page_ids[t / num_heads], head t % num_heads); invalid page ids
// are skipped.
template <int D, bool kOutF32>
__device__ __forceinline__ void summary_tile_bf16(const uint16_t* __restrict__ keys,
                                                  const int32_t* __restrict__ page_ids, int tile,
                                                  int num_pages, int num_heads, int page_size,
                                                  void* __restrict__ out) {
  constexpr int DPL = D / kWave;  // dims per lane: 1 or 2
  const int lane = threadIdx.x & 63;
  const int i = tile / num_heads, h = tile - i * num_heads;
  const int page = page_ids[i];
  if (page < 0 || page >= num_pages) return;
  const uint16_t* base = keys + ((size_t)page * num_heads + h) * (size_t)page_size * D + lane * DPL;
  double acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.0;
  for (int s = 0; s < page_size; ++s) {
    if constexpr (DPL == 2) {
      uint32_t pr = *reinterpret_cast<const uint32_t*>(base + (size_t)s * D);
      acc[0] += (double)bf16_lo(pr);
      acc[1] += (double)bf16_hi(pr);
    } else {
      acc[0] += (double)bf16_to_f32(base[(size_t)s * D]);
    }
  }
  const double inv = 1.0 / (double)page_size;  // exact: power of two
  const size_t o = ((size_t)page * num_heads + h) * D + lane * DPL;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    double mean = acc[j] * inv;
    if constexpr (kOutF32) {
      reinterpret_cast<float*>(out)[o + j] = (float)mean;  // one RNE rounding
    } else {
      reinterpret_cast<uint16_t*>(out)[o + j] = f64_to_bf16_rne(mean);
    }
  }
}

// Quest bounds of tile `tile` (as above): the element-wise maximum and
// minimum of the page's keys (Vortex, "Writing an algorithm: vFlow", Quest's
// cache step), stored as out[page][head][0][D] (maximum) and [1][D]
// (minimum). Exact: the maximum and the minimum of bf16 values are bf16
// values, so storing them is a copy of the bits. Keys are taken to be finite
// (a NaN would be skipped by the comparisons).
template <int D>
__device__ __forceinline__ void bounds_tile_bf16(const uint16_t* __restrict__ keys,
                                                 const int32_t* __restrict__ page_ids, int tile,
                                                 int num_pages, int num_heads, int page_size,
                                                 uint16_t* __restrict__ out) {
  constexpr int DPL = D / kWave;  // dims per lane: 1 or 2
  const int lane = threadIdx.x & 63;
  const int i = tile / num_heads, h = tile - i * num_heads;
  const int page = page_ids[i];
  if (page < 0 || page >= num_pages) return;
  const uint16_t* base = keys + ((size_t)page * num_heads + h) * (size_t)page_size * D + lane * DPL;
  float hi[DPL], lo[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    hi[j] = -__builtin_huge_valf();
    lo[j] = __builtin_huge_valf();
  }
  for (int s = 0; s < page_size; ++s) {
    float v[DPL];
    if constexpr (DPL == 2) {
      const uint32_t pr = *reinterpret_cast<const uint32_t*>(base + (size_t)s * D);
      v[0] = bf16_lo(pr);
      v[1] = bf16_hi(pr);
    } else {
      v[0] = bf16_to_f32(base[(size_t)s * D]);
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      hi[j] = fmaxf(hi[j], v[j]);
      lo[j] = fminf(lo[j], v[j]);
    }
  }
  uint16_t* o = out + ((size_t)page * num_heads + h) * 2 * D + lane * DPL;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    o[j] = (uint16_t)(__float_as_uint(hi[j]) >> 16);       // bf16 values: exact
    o[D + j] = (uint16_t)(__float_as_uint(lo[j]) >> 16);
  }
}

}  // namespace ls

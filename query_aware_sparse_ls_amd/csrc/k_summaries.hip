// Block summaries: the mean key of each full page, per KV head, rounded once.
//
// Vortex post, "Writing an algorithm: vFlow": the block-top-k cache step
// stores the mean of a block's keys over the in-block axis; "Why Long
// Generations Are Expensive": it runs once, when a block fills up.
//
// Layout: one wavefront per (page, head) tile. A bf16 tile is page_size rows
// of head_dim contiguous elements; lane l owns dims [l*DPL, l*DPL+DPL), so
// each row read is one coalesced 64 * DPL * 2-byte access. Sums are kept in
// float64: every bf16 value and every fp32-scale x fp8 product is exact in
// float64, so the column sum is exact unless its terms span more than ~2^41
// in magnitude; page_size is a power of two, so the mean is exact too, and it
// is rounded once (nearest-even) to the summary dtype.
#include "dev_summary.h"

namespace ls {

template <int D, bool kOutF32>
__global__ __launch_bounds__(256) void summaries_bf16_kernel(
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ page_ids, int n_pages,
    int num_pages, int num_heads, int page_size, void* __restrict__ out) {
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= n_pages * num_heads) return;
  summary_tile_bf16<D, kOutF32>(keys, page_ids, tile, num_pages, num_heads, page_size, out);
}

// fp8 e4m3fn keys with a per-token fp32 scale, single-head pool
// [num_pages][page_size][D]; the summand is scale[p][s] * key[p][s][d].
template <int D, bool kOutF32>
__global__ __launch_bounds__(256) void summaries_fp8_kernel(
    const uint8_t* __restrict__ keys, const float* __restrict__ scales,
    const int32_t* __restrict__ page_ids, int n_pages, int num_pages, int page_size,
    void* __restrict__ out) {
  constexpr int DPL = D / kWave;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tile >= n_pages) return;
  const int page = page_ids[tile];
  if (page < 0 || page >= num_pages) return;
  const uint8_t* base = keys + (size_t)page * page_size * D + lane * DPL;
  const float* sc = scales + (size_t)page * page_size;
  double acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.0;
  for (int s = 0; s < page_size; ++s) {
    const double sv = (double)sc[s];
#pragma unroll
    for (int j = 0; j < DPL; ++j)
      acc[j] += sv * (double)fp8e4m3fn_to_f32(base[(size_t)s * D + j]);  // exact product
  }
  const double inv = 1.0 / (double)page_size;
  const size_t o = (size_t)page * D + lane * DPL;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    double mean = acc[j] * inv;
    if constexpr (kOutF32) {
      reinterpret_cast<float*>(out)[o + j] = (float)mean;
    } else {
      reinterpret_cast<uint16_t*>(out)[o + j] = f64_to_bf16_rne(mean);
    }
  }
}

template <int D, bool F32>
static hipError_t launch_bf16(const SummaryArgs& a, hipStream_t st) {
  const int tiles = a.n_pages * a.pool.num_heads;
  dim3 grid((tiles + 3) / 4);
  hipLaunchKernelGGL((summaries_bf16_kernel<D, F32>), grid, dim3(256), 0, st,
                     (const uint16_t*)a.keys, a.page_ids, a.n_pages, a.pool.num_pages,
                     a.pool.num_heads, a.pool.page_size, a.out);
  return hipGetLastError();
}

template <int D, bool F32>
static hipError_t launch_fp8(const SummaryArgs& a, hipStream_t st) {
  dim3 grid((a.n_pages + 3) / 4);
  hipLaunchKernelGGL((summaries_fp8_kernel<D, F32>), grid, dim3(256), 0, st,
                     (const uint8_t*)a.keys, a.key_scales, a.page_ids, a.n_pages,
                     a.pool.num_pages, a.pool.page_size, a.out);
  return hipGetLastError();
}

template <int D>
__global__ __launch_bounds__(256) void bounds_bf16_kernel(
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ page_ids, int n_pages,
    int num_pages, int num_heads, int page_size, uint16_t* __restrict__ out) {
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= n_pages * num_heads) return;
  bounds_tile_bf16<D>(keys, page_ids, tile, num_pages, num_heads, page_size, out);
}

hipError_t launch_bounds(const SummaryArgs& a, hipStream_t st) {
  const int tiles = a.n_pages * a.pool.num_heads;
  dim3 grid((tiles + 3) / 4);
  if (a.pool.head_dim == 128)
    hipLaunchKernelGGL((bounds_bf16_kernel<128>), grid, dim3(256), 0, st,
                       (const uint16_t*)a.keys, a.page_ids, a.n_pages, a.pool.num_pages,
                       a.pool.num_heads, a.pool.page_size, (uint16_t*)a.out);
  else
    hipLaunchKernelGGL((bounds_bf16_kernel<64>), grid, dim3(256), 0, st,
                       (const uint16_t*)a.keys, a.page_ids, a.n_pages, a.pool.num_pages,
                       a.pool.num_heads, a.pool.page_size, (uint16_t*)a.out);
  return hipGetLastError();
}

hipError_t launch_summaries(const SummaryArgs& a, hipStream_t st) {
  const bool f32 = a.out_dtype == LS_DTYPE_FP32;
  const int D = a.pool.head_dim;
  if (a.pool.dtype == LS_DTYPE_BF16) {
    if (D == 128) return f32 ? launch_bf16<128, true>(a, st) : launch_bf16<128, false>(a, st);
    return f32 ? launch_bf16<64, true>(a, st) : launch_bf16<64, false>(a, st);
  }
  if (D == 128) return f32 ? launch_fp8<128, true>(a, st) : launch_fp8<128, false>(a, st);
  return f32 ? launch_fp8<64, true>(a, st) : launch_fp8<64, false>(a, st);
}

}  // namespace ls

// Block summaries: the mean key of each full page, per KV head, rounded once.
//
// Vortex post, "Writing an algorithm: vFlow": the block-top-k cache step
// stores the mean of a block's keys over the in-block axis; "Why Long
// Generations Are Expensive": it runs once, when a block fills up.
//
// Layout: one wavefront per (page, head) tile, 16-byte loads, every row of
// the tile in flight at once (the rows a lane read are summed, then the row
// groups by lane shuffles). Sums are kept in
// float64: every bf16 value and every fp32-scale x fp8 product is exact in
// float64, so the column sum is exact unless its terms span more than ~2^41
// in magnitude; page_size is a power of two, so the mean is exact too, and it
// is rounded once (nearest-even) to the summary dtype.
#include "dev_summary.h"

namespace ls {

// Standalone bf16 build: each wave takes kSumTpw consecutive (page, head)
// tiles -- a contiguous run of the pool when the page ids are -- and loads
// its next tile while it reduces the current one.
#ifndef LS_SUM_TILES_PER_WAVE
#define LS_SUM_TILES_PER_WAVE 2
#endif
#ifndef LS_SUM_WAVES
#define LS_SUM_WAVES 4
#endif
constexpr int kSumTpw = LS_SUM_TILES_PER_WAVE;
constexpr int kSumWaves = LS_SUM_WAVES;

template <int D, bool kOutF32, int PMAX>
__global__ __launch_bounds__(kSumWaves * kWave) void summaries_bf16_kernel(
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ page_ids, int n_pages,
    int num_pages, int num_heads, int page_size, void* __restrict__ out) {
  constexpr int NI = PMAX / SumTile<D>::RPI;
  const int tiles = n_pages * num_heads;
  const int t0 = (blockIdx.x * kSumWaves + (threadIdx.x >> 6)) * kSumTpw;
  // tile t's page (-1: past the end or an invalid page id)
  auto page_of = [&](int t, int* h) {
    if (t >= tiles) return -1;
    const int i = t / num_heads;
    *h = t - i * num_heads;
    const int p = page_ids[i];
    return (p >= 0 && p < num_pages) ? p : -1;
  };
  uint4 v[2][NI];
  int hh[2] = {0, 0}, pp[2];
  const int ni = page_size / SumTile<D>::RPI;
  pp[0] = page_of(t0, &hh[0]);
  if (pp[0] >= 0) (void)sum_tile_load<D, PMAX>(keys, pp[0], hh[0], num_heads, page_size, v[0]);
#pragma unroll
  for (int k = 0; k < kSumTpw; ++k) {
    const int cur = k & 1, nxt = cur ^ 1;
    if (k + 1 < kSumTpw) {
      pp[nxt] = page_of(t0 + k + 1, &hh[nxt]);
      if (pp[nxt] >= 0) (void)sum_tile_load<D, PMAX>(keys, pp[nxt], hh[nxt], num_heads, page_size, v[nxt]);
    }
    if (pp[cur] >= 0)
      summary_tile_finish<D, kOutF32, PMAX>(v[cur], ni, pp[cur], hh[cur], num_heads, page_size, out);
  }
}

// fp8 e4m3fn keys with a per-token fp32 scale, single-head pool
// [num_pages][page_size][D]; the summand is scale[p][s] * key[p][s][d]. Lane
// l loads 16 bytes (16 dims) of rows l / LPR, l / LPR + RPI, ... (LPR = D / 16
// lanes per row, RPI = 64 / LPR rows per load), all issued before the first
// use; the bytes are widened exactly with the packed convert.
template <int D, int PMAX>
struct Fp8Tile {
  static constexpr int LPR = D / 16, RPI = kWave / LPR, NI = PMAX / RPI;
  uint4 v[NI];
  float sv[NI];
};

template <int D, int PMAX>
__device__ __forceinline__ void fp8_tile_load(const uint8_t* __restrict__ keys,
                                              const float* __restrict__ scales, int page,
                                              int page_size, Fp8Tile<D, PMAX>& t) {
  using T = Fp8Tile<D, PMAX>;
  const int lane = threadIdx.x & 63;
  const int ni = page_size / T::RPI, row0 = lane / T::LPR, c = lane % T::LPR;
#pragma unroll
  for (int i = 0; i < T::NI; ++i) {
    const size_t row = (size_t)page * page_size + row0 + (size_t)i * T::RPI;
    t.v[i] = i < ni ? ldg16_stream(keys + row * D + 16 * c) : make_uint4(0, 0, 0, 0);
    t.sv[i] = i < ni ? scales[row] : 0.0f;
  }
}

template <int D, bool kOutF32, int PMAX>
__device__ __forceinline__ void fp8_tile_finish(const Fp8Tile<D, PMAX>& t, int page, int page_size,
                                                void* __restrict__ out) {
  using T = Fp8Tile<D, PMAX>;
  const int lane = threadIdx.x & 63;
  const int ni = page_size / T::RPI;
  double acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0;
#pragma unroll
  for (int i = 0; i < T::NI; ++i) {
    if (i < ni) {
      const double s = (double)t.sv[i];
      const uint32_t w[4] = {t.v[i].x, t.v[i].y, t.v[i].z, t.v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t b01 = fp8x2_to_bf16x2(w[q], false), b23 = fp8x2_to_bf16x2(w[q], true);
        acc[4 * q] += s * (double)bf16_lo(b01);       // exact products
        acc[4 * q + 1] += s * (double)bf16_hi(b01);
        acc[4 * q + 2] += s * (double)bf16_lo(b23);
        acc[4 * q + 3] += s * (double)bf16_hi(b23);
      }
    }
  }
#pragma unroll
  for (int off = T::LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] += __shfl_xor(acc[j], off, kWave);
  }
  if (lane >= T::LPR) return;
  const double inv = 1.0 / (double)page_size;
  const size_t o = (size_t)page * D + 16 * lane;
  if constexpr (kOutF32) {
    float* dst = reinterpret_cast<float*>(out) + o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(dst + 4 * q) =
          make_float4((float)(acc[4 * q] * inv), (float)(acc[4 * q + 1] * inv),
                      (float)(acc[4 * q + 2] * inv), (float)(acc[4 * q + 3] * inv));
  } else {
    uint32_t pk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pk[j] = (uint32_t)f64_to_bf16_rne(acc[2 * j] * inv) |
              ((uint32_t)f64_to_bf16_rne(acc[2 * j + 1] * inv) << 16);
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + o;
    *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
  }
}

template <int D, bool kOutF32, int PMAX>
__global__ __launch_bounds__(256) void summaries_fp8_kernel(
    const uint8_t* __restrict__ keys, const float* __restrict__ scales,
    const int32_t* __restrict__ page_ids, int n_pages, int num_pages, int page_size,
    void* __restrict__ out) {
  constexpr int kTpw = 1;   // one tile per wave (two in flight cost occupancy)
  const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kTpw;
  auto page_of = [&](int k) {
    const int t = t0 + k;
    if (t >= n_pages) return -1;
    const int p = page_ids[t];
    return (p >= 0 && p < num_pages) ? p : -1;
  };
  Fp8Tile<D, PMAX> tl[2];
  int pp[2];
  pp[0] = page_of(0);
  if (pp[0] >= 0) fp8_tile_load<D, PMAX>(keys, scales, pp[0], page_size, tl[0]);
#pragma unroll
  for (int k = 0; k < kTpw; ++k) {
    const int cur = k & 1, nxt = cur ^ 1;
    if (k + 1 < kTpw) {
      pp[nxt] = page_of(k + 1);
      if (pp[nxt] >= 0) fp8_tile_load<D, PMAX>(keys, scales, pp[nxt], page_size, tl[nxt]);
    }
    if (pp[cur] >= 0) fp8_tile_finish<D, kOutF32, PMAX>(tl[cur], pp[cur], page_size, out);
  }
}

template <int D, bool F32>
static hipError_t launch_bf16(const SummaryArgs& a, hipStream_t st) {
  const int tiles = a.n_pages * a.pool.num_heads;
  const int per = kSumWaves * kSumTpw;
  dim3 grid((tiles + per - 1) / per);
  const int P = a.pool.page_size;
#define LS_SUM_LAUNCH(PM)                                                                    \
  hipLaunchKernelGGL((summaries_bf16_kernel<D, F32, PM>), grid, dim3(kSumWaves * kWave), 0, st,           \
                     (const uint16_t*)a.keys, a.page_ids, a.n_pages, a.pool.num_pages,      \
                     a.pool.num_heads, P, a.out)
  if (P <= 16) LS_SUM_LAUNCH(16);
  else if (P <= 32) LS_SUM_LAUNCH(32);
  else LS_SUM_LAUNCH(64);
#undef LS_SUM_LAUNCH
  return hipGetLastError();
}

template <int D, bool F32>
static hipError_t launch_fp8(const SummaryArgs& a, hipStream_t st) {
  dim3 grid((a.n_pages + 3) / 4);
  const int P = a.pool.page_size;
#define LS_FP8_LAUNCH(PM)                                                                    \
  hipLaunchKernelGGL((summaries_fp8_kernel<D, F32, PM>), grid, dim3(256), 0, st,            \
                     (const uint8_t*)a.keys, a.key_scales, a.page_ids, a.n_pages,           \
                     a.pool.num_pages, P, a.out)
  if (P <= 16) LS_FP8_LAUNCH(16);
  else if (P <= 32) LS_FP8_LAUNCH(32);
  else LS_FP8_LAUNCH(64);
#undef LS_FP8_LAUNCH
  return hipGetLastError();
}

template <int D, int PMAX>
__global__ __launch_bounds__(256) void bounds_bf16_kernel(
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ page_ids, int n_pages,
    int num_pages, int num_heads, int page_size, uint16_t* __restrict__ out) {
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= n_pages * num_heads) return;
  bounds_tile_bf16<D, PMAX>(keys, page_ids, tile, num_pages, num_heads, page_size, out);
}

template <int D>
static hipError_t launch_bounds_d(const SummaryArgs& a, hipStream_t st) {
  const int tiles = a.n_pages * a.pool.num_heads;
  dim3 grid((tiles + 3) / 4);
  const int P = a.pool.page_size;
#define LS_BND_LAUNCH(PM)                                                                    \
  hipLaunchKernelGGL((bounds_bf16_kernel<D, PM>), grid, dim3(256), 0, st,                    \
                     (const uint16_t*)a.keys, a.page_ids, a.n_pages, a.pool.num_pages,      \
                     a.pool.num_heads, P, (uint16_t*)a.out)
  if (P <= 16) LS_BND_LAUNCH(16);
  else if (P <= 32) LS_BND_LAUNCH(32);
  else LS_BND_LAUNCH(64);
#undef LS_BND_LAUNCH
  return hipGetLastError();
}

hipError_t launch_bounds(const SummaryArgs& a, hipStream_t st) {
  return a.pool.head_dim == 128 ? launch_bounds_d<128>(a, st) : launch_bounds_d<64>(a, st);
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

// Learned-indexer scoring and token top-k (device code).
//
// Score of a unit u (a token of the indexer key pool, or a block through its
// block-mean indexer key) for request r (LeanSparse, Eq. 6 with the original
// keys; coarse pass on block means):
//     s_u = sum_h w[r][h] * max(0, sigma_u * (q[r][h] . key_u))
// with q bf16 [B][H][128], w fp32 [B][H], key_u fp8 e4m3fn (token mode, with
// per-token scale sigma_u) or bf16 (block mode, sigma = 1).
//
// The contraction q . key over 128 dims for H = 16..64 heads is a dense GEMM
// per 16-unit tile: one v_mfma_f32_16x16x32_bf16 per (16-head tile, 32-dim
// k-step) with A = q (rows = heads) and B = key^T (columns = units), so each
// lane ends up with one unit's 4 heads per head tile. fp8 keys are widened to
// bf16 exactly (every e4m3fn value is a bf16 value) with the gfx950 convert
// instruction; products of bf16 and fp8 values are exact in fp32 and the
// MFMA accumulates in fp32.
//
// Operand layout. Keys are loaded from memory row-major, 1 KB contiguous per
// wave instruction, staged in a padded LDS tile per wave, and read back as
// lane i <- unit row i%16, 32 bytes (fp8) or 64 bytes (bf16) of dims starting
// at 32(i/16). K-step s of the MFMA then uses dims 32(i/16) + 8s .. + 8 of
// that slice; the q operand is loaded with the same dim permutation, which
// leaves every dot product unchanged (the sum over dims is over the same
// pairs).
//
// Token top-k (k of up to 262,144 units per request, ties to the lowest unit).
// The first digit is a bucket of a monotonic remap of the scores (Vortex
// post, "Making it fast": the remap spreads the scores over the buckets):
// linear from the request's smallest to its largest valid score onto 4,096
// buckets, so that the bucket holding the k-th score holds few units; the
// units that share the k-th score's first digit are then ranked by an
// order-preserving integer key of their fp32 scores:
//  1. every scoring workgroup leaves the (min, max) of its valid scores in a
//     slot (workgroup 0 of a request also clears the request's histogram and
//     counters);
//  2. the histogram kernel reduces the request's slots to the remap, and
//     histograms the first digit (bucket >> 4: 256 bins, so that every
//     workgroup adds at most 256 counts into the request's global histogram
//     with device-scope atomics);
//  3. the mark kernel finds, per request, the first digit d* holding the
//     k-th score; units above d* are selected (bitmap), units of d* are
//     appended to a per-request list;
//  4. the last mark workgroup of each request (arrival counter) ranks the
//     listed units: up to 512 of them directly in LDS, by (key descending,
//     unit ascending), more of them by three digits of their key (12, 12, 8
//     bits); it marks the winners and emits the bitmap in ascending order.
//     The approximate top-k ranks the listed units by their bucket instead
//     of their key (an early exit at bucket resolution: the bucket holding
//     the k-th score is filled in ascending unit order).
#pragma once

#include "ls_internal.h"

namespace ls {

constexpr int kIdxDim = 128;            // indexer key / query dim
constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / kWave;
#ifndef LS_IDX_PREFETCH
#define LS_IDX_PREFETCH 4
#endif
constexpr int kIdxPrefetch = LS_IDX_PREFETCH;   // key tiles in flight per wave
constexpr int kIdxMaxTilesPerWg = 128;  // units per scoring workgroup <= 2048
constexpr int kIdxMaxWords = kIdxMaxUnits / 32;

// Units of request r in token mode: without candidates, the cached tokens
// [0, L); with candidates, n_c blocks of P units each (unit u = slot u % P of
// candidate block u / P), valid when the block id is valid and the token is
// cached.
// With token candidates (unit_kind kUnitsTokenCands) unit u < n_c is token
// cand[u] and unit n_c + i is token tail0 + i of the partial last page; with
// kUnitsComplete the units are the tokens [0, tail0) of the complete pages.
struct IdxUnits {
  int n;          // units (valid or not) of the request
  int L, nb, page_base;
  int ncand;      // -1: no candidate list
  int tail0;      // first token of the partial last page (= L when none)
};

__device__ __forceinline__ IdxUnits idx_units(const IndexerArgs& a, int r) {
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  IdxUnits u;
  u.L = geo.L;
  u.nb = geo.nb;
  u.page_base = geo.page_base;
  u.tail0 = geo.L & ~(a.b.page_size - 1);   // a power of two
  if (a.unit_kind == kUnitsTokenCands) {
    int c = a.cand_counts[r];
    c = c < 0 ? 0 : (c > a.cand_cap ? a.cand_cap : c);
    u.ncand = c;
    u.n = c + (geo.L - u.tail0);
  } else if (a.unit_kind == kUnitsComplete) {
    u.ncand = -1;
    u.n = u.tail0;
  } else if (a.cand_blocks) {
    int c = a.cand_counts[r];
    c = c < 0 ? 0 : (c > a.cand_cap ? a.cand_cap : c);
    u.ncand = c;
    u.n = c * a.b.page_size;
  } else {
    u.ncand = -1;
    u.n = geo.L;
  }
  if (u.n > a.max_units) u.n = a.max_units;
  return u;
}

// Block of unit u (token mode) or -1 when the unit is not a cached token.
__device__ __forceinline__ int idx_unit_block(const IndexerArgs& a, const IdxUnits& g, int r,
                                              int u, int* token) {
  const int P = a.b.page_size, PS = __builtin_ctz((unsigned)P);   // a power of two
  if (u < 0 || u >= g.n) return -1;
  if (a.unit_kind == kUnitsTokenCands) {
    const int t = u < g.ncand ? a.cand_blocks[(size_t)r * a.cand_cap + u] : g.tail0 + (u - g.ncand);
    if (t < 0 || t >= g.L) return -1;
    *token = t;
    return t >> PS;
  }
  int blk;
  if (g.ncand < 0) {
    blk = u >> PS;
  } else {
    blk = a.cand_blocks[(size_t)r * a.cand_cap + (u >> PS)];
    if (blk < 0 || blk >= g.nb) return -1;
  }
  const int t = blk * P + (u & (P - 1));
  if (t >= g.L) return -1;
  *token = t;
  return blk;
}

// The remap: scale = kIdxBins / (mx - mn) in fp32, rounded once; 0 when the
// range is empty, negative or not finite (every unit in bucket 0).
__device__ __forceinline__ float idx_remap_scale(float mn, float mx) {
  const float span = mx - mn;
  if (!(span > 0.0f) || !(span <= 3.402823466e38f)) return 0.0f;   // NaN fails both
  return __fdiv_rn((float)kIdxBins, span);
}

// Bucket of score s: t = (s - mn) * scale, each step rounded once; the top
// bucket takes t >= kIdxBins - 1 (the largest score lands on kIdxBins), and a
// NaN t bucket 0.
__device__ __forceinline__ int idx_remap_bin(float s, float mn, float scale) {
  const float t = (s - mn) * scale;
  return t >= (float)(kIdxBins - 1) ? kIdxBins - 1 : (t >= 1.0f ? (int)t : 0);
}

// (min, max) over the workgroup of each thread's (mn, mx); every thread gets
// the result. red: 2 * waves floats of LDS. Synchronises.
template <int NT>
__device__ __forceinline__ void idx_range_reduce(float& mn, float& mx, float* red) {
  constexpr int NW = NT / kWave;
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[wave] = mn;
    red[NW + wave] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    mn = fminf(mn, red[w]);
    mx = fmaxf(mx, red[NW + w]);
  }
  __syncthreads();
}

// Workgroup 0 of request r clears the request's histogram and counters
// before the histogram kernel (a later launch) uses them.
template <int NT>
__device__ __forceinline__ void idx_clear_request(const IndexerArgs& a, int r) {
  uint4* h = reinterpret_cast<uint4*>(a.hist + (size_t)r * kIdxCoarse);
  for (int i = threadIdx.x; i < kIdxCoarse / 4; i += NT) h[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < 4) a.ctl[(size_t)r * 4 + threadIdx.x] = 0u;
}

// max(x, 0) as one integer max on the bits: a negative float (sign bit set)
// is a negative int and becomes +0; anything else is kept (NaN included).
__device__ __forceinline__ float relu_bits(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

}  // namespace ls

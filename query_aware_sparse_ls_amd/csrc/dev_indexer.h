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
// Token top-k (k of up to 262,144 units per request, ties to the lowest unit),
// a three-digit radix select over an order-preserving integer key of the
// scores:
//  1. the scoring workgroups histogram the key's top 12 bits in LDS and add
//     the non-zero bins into a per-request global histogram (device-scope
//     atomics);
//  2. the mark kernel finds, per request, the bucket b* holding the k-th
//     score; units above b* are selected (bitmap), units in b* are appended
//     to a per-request list and histogrammed by their next 12 key bits;
//  3. the last mark workgroup of each request (arrival counter) finds the
//     second digit from that histogram, the third (last 8 bits) in one pass
//     over the list, marks the listed units above the k-th key, takes the
//     ones equal to it lowest index first, and emits the bitmap in ascending
//     order.
#pragma once

#include "ls_internal.h"

namespace ls {

constexpr int kIdxDim = 128;            // indexer key / query dim
constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kIdxPrefetch = 2;         // key tiles in flight per wave
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

__device__ __forceinline__ uint32_t idx_bin(uint32_t key) { return key >> 20; }

// max(x, 0) as one integer max on the bits: a negative float (sign bit set)
// is a negative int and becomes +0; anything else is kept (NaN included).
__device__ __forceinline__ float relu_bits(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

}  // namespace ls

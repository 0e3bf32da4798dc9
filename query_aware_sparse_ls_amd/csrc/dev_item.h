// Per-(request, kv head) workgroup code: ONE 512-thread workgroup owns a whole
// (request r, kv head g) pair and runs its steps back to back -- block scoring
// into LDS, top-k from LDS, attention over the selection with the merge of
// all partial softmax states in LDS. Nothing is handed between workgroups, so
// there are no split partials, arrival counters or extra launches.
//
// Both contractions run on the matrix cores (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x16_bf16). For a 16-row tile of keys K (summary rows or the
// 16 tokens of a block) and the GQA group's G = 4 query heads, the product
// K . Q^T is a 16 x 16 MFMA whose 16 columns are the query heads, zero-padded
// from 4; the vector ALU alone cannot keep up with HBM here (about 50 VALU
// wave-instructions per 512 bytes of K and V at G = 4, against the ~10 bytes
// per wave-instruction the chip's VALU rate allows at full bandwidth).
//  * K operand: lane i holds row i%16, dims [32j + 8(i/16), +8) of k-step j.
//    Rows are loaded from memory in the plain row-major order instead (each
//    wave load instruction reads 1 KB contiguous: whole 128-byte lines), and
//    reach the operand layout through a padded LDS tile per wave: loading the
//    operand layout directly (16 rows x 64 B per instruction) measured about
//    1.6x slower on this chip, and worse the more loads are in flight.
//  * Q^T operand: lane i holds q[head i%16][the same dims] (0 for head >= 4).
//  * Output: lane i holds head i%16 for rows 4(i/16) .. 4(i/16)+3.
// The attention output P . V is a 16 x 16 x 16 MFMA per 16 output dims with P
// (heads x tokens) in exactly that output layout, and V (tokens x dims) as
// the B operand: lane i needs 4 tokens of one dim, a column of the row-major
// V tile, gathered from the wave's LDS copy of the tile with one transpose
// read (ds_read_b64_tr_b16) per 16-dim tile. P is split into bf16 parts, p = hi + lo (+ lo2
// for fp32 output), so the products keep fp32-level accuracy.
#pragma once

#include "dev_attn.h"
#include "dev_mfma.h"
#include "dev_score.h"
#include "dev_topk.h"

namespace ls {

constexpr int kItemThreads = 512;
constexpr int kItemWaves = kItemThreads / kWave;
constexpr int kItemScorePrefetch = 2;   // summary tiles in flight per wave
constexpr int kItemBoundsPrefetch = 1;  // bounds tiles (max + min rows) in flight per wave
constexpr int kItemPrefetch = 2;        // K/V blocks in flight per wave
// Walk entries past the selection that item_attn may read: wave w refills
// its slots with position w + 8(k + kItemPrefetch) for k < nbw + kItemPrefetch
// - 1, nbw = ceil((cnt - w) / 8), i.e. at most cnt + 7 + 8(2 kItemPrefetch - 2).
template <int NW>
constexpr int item_entry_pad() { return NW * 2 * kItemPrefetch; }
constexpr int kItemEntryPad = item_entry_pad<kItemWaves>();
static_assert(kItemEntryPad >= 7 + kItemWaves * (2 * kItemPrefetch - 2) + 1, "entry padding");

// Where item_score / item_score_bounds put the scores: every row of the
// scored tiles into LDS, or the candidate rows into a global score row with
// plain stores (read by a later launch) or device-coherent stores (read by
// another workgroup of the same launch); kStoreDevKey stores the
// order-preserving key of the score (score_key, never 0 for a finite score)
// as a uint32, so that a zero word means "not written yet".
enum { kStoreLds = 0, kStoreGlobal = 1, kStoreDev = 2, kStoreDevKey = 3 };

// How item_attn writes a split's state: plain stores, device-coherent
// stores, or device-coherent stores of the bitwise complement (never 0 for
// a finite value: a zero word means "not written yet").
enum { kSplitPlain = 0, kSplitDev = 1, kSplitDevEnc = 2 };

template <int kMode>
__device__ __forceinline__ void store_split_word(float* p, float v) {
  if constexpr (kMode == kSplitDevEnc)
    st_dev(reinterpret_cast<uint32_t*>(p), ~__float_as_uint(v));
  else
    st_x<kMode == kSplitDev>(p, v);
}

// The 4 group queries as a 16x16x32 MFMA operand, one per k-step of D/32:
// lane i holds head i%16 (zero past the 4 heads), dims 32j + 8(i/16) .. +8.
// The A and B operands take the same lane layout, so the same registers
// serve as Q (A: rows = heads) or Q^T (B: columns = heads).
template <int D>
struct QOperand {
  uint4 b[D / 32];
};

template <int D>
__device__ __forceinline__ QOperand<D> load_q_operand(const uint16_t* q, int num_q_heads, int r,
                                                      int g) {
  const int lane = threadIdx.x & 63, h = lane & 15, kq = lane >> 4;
  QOperand<D> o;
  const uint16_t* qh = q + ((size_t)r * num_q_heads + g * 4 + (h < 4 ? h : 0)) * D + 8 * kq;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) o.b[j] = h < 4 ? ldg16(qh + 32 * j) : make_uint4(0, 0, 0, 0);
  return o;
}

// Page ids of blocks [0, nb) of request r into pg[] (LDS; nb <= MAXC); the
// caller synchronises before use. One coalesced pass over the page-table
// row, every load of a thread issued before its stores.
template <int MAXC>
__device__ __forceinline__ void load_page_row(const BatchArgs& b, const ReqGeom& geo, int* pg) {
  constexpr int NPT = (MAXC + kItemThreads - 1) / kItemThreads;
  int v[NPT];
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int i = threadIdx.x + m * kItemThreads;
    v[m] = i < geo.nb ? b.indices[geo.page_base + i] : 0;
  }
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int i = threadIdx.x + m * kItemThreads;
    if (i < geo.nb) pg[i] = v[m];
  }
}

// Row-major staging of a 16 x D bf16 tile: lane i loads rows j*RPI + i/LPR,
// 16 bytes at dims 8(i%LPR) (LPR = D/8 lanes per row, RPI = 64/LPR rows per
// instruction, D/32 instructions for 16 rows).
template <int D>
struct Stage {
  static constexpr int LPR = D / 8, RPI = kWave / LPR, NL = D / 32;
  static constexpr int kKRowWords = D / 2 + 4;   // K tile rows: 16-byte aligned, padded
  static constexpr int kVRowWords = D / 2 + 8;   // V tile rows: the 4 rows of a transpose read hit 32 distinct banks
};

// Writes this lane's NL row chunks into a K-style LDS tile (row stride
// kKRowWords words); zero = write zeros instead.
template <int D>
__device__ __forceinline__ void stage_k(uint32_t* tile, const uint4* d, uint32_t zero_mask) {
  using S = Stage<D>;
  const int lane = threadIdx.x & 63;
  uint32_t* dst = tile + (lane / S::LPR) * S::kKRowWords + 4 * (lane % S::LPR);
  if (__ballot(zero_mask != 0u) == 0) {   // the common case: nothing to clear
#pragma unroll
    for (int j = 0; j < S::NL; ++j)
      *reinterpret_cast<uint4*>(dst + j * S::RPI * S::kKRowWords) = d[j];
  } else {
#pragma unroll
    for (int j = 0; j < S::NL; ++j)
      *reinterpret_cast<uint4*>(dst + j * S::RPI * S::kKRowWords) =
          ((zero_mask >> j) & 1u) ? make_uint4(0, 0, 0, 0) : d[j];
  }
}

// The MFMA operand of k-step j from a K-style LDS tile: row i%16, dims
// [32j + 8(i/16), +8) -- the tile as A (rows = tile rows) or as B (columns =
// tile rows, i.e. the tile transposed).
template <int D>
__device__ __forceinline__ uint4 k_operand(const uint32_t* tile, int j) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const uint4*>(tile + (lane & 15) * Stage<D>::kKRowWords + 16 * j +
                                         4 * (lane >> 4));
}

// s[b] for every candidate block b in [c0, c1) of (r, g) into sc[] (LDS), from
// the page ids in pg[] (LDS). Tile t = summary rows of blocks [16t, 16t+16);
// wave w scores tiles w, w + 8, ... of the candidate range, keeping
// kItemScorePrefetch tiles of loads in flight (each slot is refilled right
// after its use; every load is issued -- a row outside the candidates reads
// page 0 and is discarded -- so the number in flight is fixed). A candidate
// whose page id is out of range scores 0.
// pg[b - pg_off] is the page id of candidate b; NW waves take the tiles.
template <int D, int MAXC, int kStore = kStoreLds, int NW = kItemWaves,
          int NS = kItemScorePrefetch>
__device__ __forceinline__ void item_score(const ScoreArgs& a, int r, int g, const ReqGeom& geo,
                                           const int* pg, float* sc, uint32_t* stage,
                                           float* range = nullptr, int pg_off = 0) {
  using ST = Stage<D>;
  constexpr int KS = D / 32, NL = ST::NL;
  static_assert(NS % 2 == 0, "slots are consumed in pairs");
  const int HKV = a.num_kv_heads;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  const QOperand<D> qo = load_q_operand<D>(a.q, a.num_q_heads, r, g);
  const uint16_t* base = a.summaries + (size_t)g * D + 8 * (lane % ST::LPR);
  const uint32_t pstride = (uint32_t)HKV * D;   // elements per page (< 2^32)
  uint32_t* tiles = stage + wave * 2 * 16 * ST::kKRowWords;   // two tiles per wave
  const int t0 = geo.c0 / 16, t1 = (geo.c1 + 15) / 16;
  const int ntw = t1 - t0 > wave ? (t1 - t0 - wave + NW - 1) / NW : 0;
  // page of the row this lane loads with instruction j of the wave's k-th
  // tile: -1 if not a candidate, -2 for a candidate with a bad page id
  auto page_of = [&](int k, int j) {
    const int b = (t0 + wave + NW * k) * 16 + j * ST::RPI + lane / ST::LPR;
    if (k >= ntw || b < geo.c0 || b >= geo.c1) return -1;
    const int p = pg[b - pg_off];   // b in [c0, c1): inside the caller's page list
    return (p >= 0 && p < a.b.num_pages) ? p : -2;
  };
  auto issue = [&](int k, uint4* d, uint32_t& badm) {
    badm = 0;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int p = page_of(k, j);
      badm |= (uint32_t)(p == -2) << j;
      d[j] = ldg16_stream(base + (uint64_t)(uint32_t)(p >= 0 ? p : 0) * pstride);
    }
  };
  // score the staged tile and store the candidate rows (tiles past the
  // wave's range hold page-0 rows and store nothing)
  // The logits come out as D[head][token] (A = the queries, B = the tile's
  // rows as K^T): lanes 0..15 hold heads 0..3 of token `row` in acc[0..3], so
  // the group aggregation is lane-local and the 16 lanes store the tile's 16
  // scores with one LDS write. The LDS form stores non-candidate rows too
  // (the top-k reads only [c0, c1), and tile ends stay below MAXC).
  static_assert(MAXC % 16 == 0, "whole score tiles");
  const bool mean = a.group_agg == LS_AGG_MEAN;
  // this lane's smallest and largest candidate score (for range[])
  float smin = __builtin_huge_valf(), smax = -__builtin_huge_valf();
  auto finish = [&](const f32x4_t& acc, int k) {
    const float v = mean ? ((acc[0] + acc[1]) + (acc[2] + acc[3])) * 0.25f
                         : fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    if (kq == 0 && k < ntw) {
      const int b = (t0 + wave + NW * k) * 16 + row;
      const bool cand = b >= geo.c0 && b < geo.c1;
      if constexpr (kStore == kStoreLds) sc[b] = v;
      else if constexpr (kStore == kStoreDevKey) {
        if (cand) st_dev(reinterpret_cast<uint32_t*>(sc) + b, score_key(v));
      } else if (cand) st_x<kStore == kStoreDev>(&sc[b], v);
      smin = cand ? fminf(smin, v) : smin;
      smax = cand ? fmaxf(smax, v) : smax;
    }
  };
  uint4 buf[NS][NL];
  uint32_t badm[NS];   // per slot: bit j = this lane's row of instruction j has a bad page
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    issue(s, buf[s], badm[s]);
    __builtin_amdgcn_sched_barrier(0);   // issue the slots in order (oldest = slot 0)
  }
  for (int k0 = 0; k0 < ntw; k0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; s += 2) {
      // take two slots' rows and refill both at once; the two tiles are then
      // scored as independent chains, so their LDS and MFMA latencies overlap
      uint4 c0[NL], c1[NL];
      const uint32_t b0 = badm[s], b1 = badm[s + 1];
#pragma unroll
      for (int j = 0; j < NL; ++j) { c0[j] = buf[s][j]; c1[j] = buf[s + 1][j]; }
      __builtin_amdgcn_sched_barrier(0);
      issue(k0 + s + NS, buf[s], badm[s]);
      issue(k0 + s + 1 + NS, buf[s + 1], badm[s + 1]);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t* ta = tiles;
      uint32_t* tb = tiles + 16 * ST::kKRowWords;
      stage_k<D>(ta, c0, b0);   // rows with a bad page score 0
      stage_k<D>(tb, c1, b1);
      f32x4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        acc0 = mfma_16x16x32(qo.b[j], k_operand<D>(ta, j), acc0);
        acc1 = mfma_16x16x32(qo.b[j], k_operand<D>(tb, j), acc1);
      }
      // acc[i] = q_h . k of tile row `row` for head h = 4kq + i
      finish(acc0, k0 + s);
      finish(acc1, k0 + s + 1);
    }
  }
  if (range) {   // range[wave] = the wave's smallest score, range[NW + wave] its largest
    smin = wave_min_fast(smin);
    smax = wave_max_fast(smax);
    if (lane == 0) {
      range[wave] = smin;
      range[NW + wave] = smax;
    }
  }
}

// Quest bound scores (Vortex, "Writing an algorithm: vFlow", the Quest
// listing) of the candidate blocks of (r, g) into sc[] (LDS), from the bounds
// pool [num_pages][Hkv][2][D] (maximum row, then minimum row):
//     u_h(b) = sum_d max(q_hd * max_bd, q_hd * min_bd)
//            = q_h+ . max_b + q_h- . min_b,  q+ = max(q, 0), q- = min(q, 0)
// (max_bd >= min_bd, so q_hd >= 0 picks the maximum and q_hd < 0 the
// minimum), i.e. two dense contractions: each k-step runs one MFMA with the
// staged maximum rows and one with the minimum rows. q+ and q- are bf16
// values (q or 0), the products are exact in fp32. The group aggregation,
// score stores and range are those of item_score; one slot holds both rows
// of a 16-block tile.
template <int D, int MAXC, int kStore = kStoreLds, int NW = kItemWaves>
__device__ __forceinline__ void item_score_bounds(const ScoreArgs& a, int r, int g,
                                                  const ReqGeom& geo, const int* pg, float* sc,
                                                  uint32_t* stage, float* range = nullptr,
                                                  int pg_off = 0) {
  using ST = Stage<D>;
  constexpr int KS = D / 32, NL = ST::NL, NS = kItemBoundsPrefetch;
  const int HKV = a.num_kv_heads;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row = lane & 15, kq = lane >> 4;
  QOperand<D> qp = load_q_operand<D>(a.q, a.num_q_heads, r, g), qn;
  // q- keeps the negative bf16 halves, q+ the others (by the sign bit)
  auto split = [](uint32_t w, uint32_t* pos) {
    const uint32_t neg = ((w & 0x80008000u) >> 15) * 0xFFFFu;
    *pos = w & ~neg;
    return w & neg;
  };
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    uint4& b = qp.b[j];
    uint4 nb;
    nb.x = split(b.x, &b.x);
    nb.y = split(b.y, &b.y);
    nb.z = split(b.z, &b.z);
    nb.w = split(b.w, &b.w);
    qn.b[j] = nb;
  }
  const uint16_t* base = a.summaries + (size_t)g * 2 * D + 8 * (lane % ST::LPR);
  const uint32_t pstride = (uint32_t)HKV * 2 * D;   // elements per page (< 2^32)
  uint32_t* tiles = stage + wave * 2 * 16 * ST::kKRowWords;   // maximum rows, minimum rows
  const int t0 = geo.c0 / 16, t1 = (geo.c1 + 15) / 16;
  const int ntw = t1 - t0 > wave ? (t1 - t0 - wave + NW - 1) / NW : 0;
  auto page_of = [&](int k, int j) {
    const int b = (t0 + wave + NW * k) * 16 + j * ST::RPI + lane / ST::LPR;
    if (k >= ntw || b < geo.c0 || b >= geo.c1) return -1;
    const int p = pg[b - pg_off];   // b in [c0, c1): inside the caller's page list
    return (p >= 0 && p < a.b.num_pages) ? p : -2;
  };
  // slot layout: d[j] = maximum-row chunk j, d[NL + j] = minimum-row chunk j
  auto issue = [&](int k, uint4* d, uint32_t& badm) {
    badm = 0;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int p = page_of(k, j);
      badm |= (uint32_t)(p == -2) << j;
      const uint16_t* rp = base + (uint64_t)(uint32_t)(p >= 0 ? p : 0) * pstride;
      d[j] = ldg16_stream(rp);
      d[NL + j] = ldg16_stream(rp + D);
    }
  };
  static_assert(MAXC % 16 == 0, "whole score tiles");
  const bool mean = a.group_agg == LS_AGG_MEAN;
  float smin = __builtin_huge_valf(), smax = -__builtin_huge_valf();
  auto finish = [&](const f32x4_t& acc, int k) {
    const float v = mean ? ((acc[0] + acc[1]) + (acc[2] + acc[3])) * 0.25f
                         : fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    if (kq == 0 && k < ntw) {
      const int b = (t0 + wave + NW * k) * 16 + row;
      const bool cand = b >= geo.c0 && b < geo.c1;
      if constexpr (kStore == kStoreLds) sc[b] = v;
      else if constexpr (kStore == kStoreDevKey) {
        if (cand) st_dev(reinterpret_cast<uint32_t*>(sc) + b, score_key(v));
      } else if (cand) st_x<kStore == kStoreDev>(&sc[b], v);
      smin = cand ? fminf(smin, v) : smin;
      smax = cand ? fmaxf(smax, v) : smax;
    }
  };
  uint4 buf[NS][2 * NL];
  uint32_t badm[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    issue(s, buf[s], badm[s]);
    __builtin_amdgcn_sched_barrier(0);   // issue the slots in order (oldest = slot 0)
  }
  for (int k0 = 0; k0 < ntw; k0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 c[2 * NL];
      const uint32_t bm = badm[s];
#pragma unroll
      for (int j = 0; j < 2 * NL; ++j) c[j] = buf[s][j];
      __builtin_amdgcn_sched_barrier(0);
      issue(k0 + s + NS, buf[s], badm[s]);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t* thi = tiles;
      uint32_t* tlo = tiles + 16 * ST::kKRowWords;
      stage_k<D>(thi, c, bm);        // rows with a bad page score 0
      stage_k<D>(tlo, c + NL, bm);
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        acc = mfma_16x16x32(qp.b[j], k_operand<D>(thi, j), acc);
        acc = mfma_16x16x32(qn.b[j], k_operand<D>(tlo, j), acc);
      }
      finish(acc, k0 + s);
    }
  }
  if (range) {
    smin = wave_min_fast(smin);
    smax = wave_max_fast(smax);
    if (lane == 0) {
      range[wave] = smin;
      range[NW + wave] = smax;
    }
  }
}

// LDS of the attention: per-wave K and V staging tiles and the wave states.
// A wave's o accumulator (4 heads x D floats) goes into its own K tile once
// its walk is done (acc_of), so the merge needs no space of its own.
template <int D, int NW = kItemWaves>
struct alignas(16) ItemAttnLds {   // 16-byte aligned: the tiles take 16-byte LDS accesses
  alignas(16) uint32_t k[NW][16 * Stage<D>::kKRowWords];
  alignas(16) uint32_t v[NW][16 * Stage<D>::kVRowWords];
  float m[NW][4];
  float l[NW][4];
  static_assert(4 * D <= 16 * Stage<D>::kKRowWords, "o accumulator fits a K tile");
  __device__ float* acc_of(int w) { return reinterpret_cast<float*>(k[w]); }
};

// Rewrites the selection sel[0 .. npad) (LDS) in place into walk entries:
// e = page * 32 + (valid tokens of the block) for positions < cnt whose block
// and page are valid, -1 otherwise. Requires num_pages < 2^26.
template <int NT = kItemThreads>
__device__ __forceinline__ void item_entries(const AttnArgs& a, const ReqGeom& geo, int* sel,
                                             int cnt, const int* pg, int npad) {
  for (int pos = threadIdx.x; pos < npad; pos += NT) {
    int e = -1;
    if (pos < cnt) {
      const int blk = sel[pos];
      if (blk >= 0 && blk < geo.nb) {
        const int p = pg[blk];
        const int nt = geo.L - blk * 16 < 16 ? geo.L - blk * 16 : 16;
        if (p >= 0 && p < a.b.num_pages && nt > 0) e = p * 32 + nt;
      }
    }
    sel[pos] = e;
  }
}

// Number of walk entries item_attn reads for a selection of cnt blocks.
template <int NW = kItemWaves>
__device__ __forceinline__ int item_entry_count(int cnt) { return cnt + item_entry_pad<NW>(); }

// Attention of the G = 4 query heads of (r, g) over the walk entries ent[]
// (LDS, from item_entries; cnt = selection size), written as out / lse.
// Wave w takes selection positions w, w + 8, ...; per block it computes the
// 16 x 4 logits with D/32 MFMAs, updates its per-head softmax state (max m,
// sum l; the o accumulator is rescaled only when a head's max grows), and
// adds P . V with D/16 MFMAs per bf16 part of P. Blocks are prefetched
// kItemPrefetch ahead per wave. The 8 wave states are merged in LDS in wave
// order.
// Floats of a pair's exchange area (two merged states of 4 heads: o, then m, l).
template <int D>
constexpr int kPairFloats = 2 * 4 * D + 16;

// Exchange area of a (request, kv head) pair whose selection is attended by
// two workgroups: each publishes its merged state (o[4][D], m[4], l[4]) and
// the second to arrive merges both and writes the output.
struct ItemPair {
  float* part;         // [2][4][D] o, then [2][4][2] (m, l)
  uint32_t* arrivals;  // zero before the launch
  int half;            // which of the two workgroups this is
};

// Elements of the merged state each thread of an NW-wave workgroup holds:
// element e = tid + j * NW * 64 (head e / D, dim e % D), j < item_ept.
template <int D, int NW>
constexpr int item_ept() { return (4 * D + NW * kWave - 1) / (NW * kWave); }

// The merged state of the positions item_attn walked, in the element layout
// above: o relative to the maximum, m (log2 domain) and l per element's
// head. Given to item_attn, it receives the state instead of any store.
template <int EPT>
struct ItemState {
  float m[EPT], o[EPT], l[EPT];
};

// Split s of num_splits of a (request, kv head) pair's positions: the merged
// state is written unnormalised as split s of the split-K partials
// (o relative to the split maximum, then m in the log2 domain, then l; the
// layout attn_split writes), for the combine kernel to merge.
struct ItemSplit {
  float* part;
  int num_splits;
  int s;
};

// kLo: entries carry a first valid token too (e = page * 512 + lo * 32 +
// nt: tokens lo .. nt-1 of the block are attended; page < 2^22), for token
// ranges that start inside a block.
// NW: waves of the workgroup; NPF: K/V blocks in flight per wave (at most
// kItemPrefetch). kSplitStore: how the split state is written (kSplit*).
template <int D, bool kLo = false, int NW = kItemWaves, int kSplitStore = kSplitPlain,
          int NPF = kItemPrefetch>
__device__ __forceinline__ void item_attn(const AttnArgs& a, int r, int g, const int* ent,
                                          int cnt, ItemAttnLds<D, NW>& sh,
                                          const ItemPair* pair = nullptr,
                                          const ItemSplit* split = nullptr,
                                          ItemState<item_ept<D, NW>()>* state = nullptr) {
  using ST = Stage<D>;
  constexpr int KS = D / 32, NL = ST::NL, NT = D / 16;
  // (entry reads past the written ones are guarded: any depth is safe)
  static_assert(NPF >= 1 && NPF <= 4, "K/V blocks in flight per wave");
  constexpr int RW = ST::kVRowWords;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int row = lane & 15, kq = lane >> 4;
  const bool head_lane = row < 4;
  cnt = __builtin_amdgcn_readfirstlane(cnt);   // uniform over the workgroup
  const int HKV = a.num_kv_heads;
  const bool out32 = a.out_dtype == LS_DTYPE_FP32;
  const QOperand<D> qo = load_q_operand<D>(a.q, a.num_q_heads, r, g);
  const uint32_t pstride = (uint32_t)HKV * 16 * D;   // elements per page (< 2^32)
  // row-major loads: instruction j reads tile rows j*RPI + lane/LPR
  const size_t lofs = ((size_t)g * 16 + lane / ST::LPR) * D + 8 * (lane % ST::LPR);
  const uint16_t* kb = a.k_pool + lofs;
  const uint16_t* vb = a.v_pool + lofs;
  uint32_t* kt = sh.k[wave];
  uint32_t* vt = sh.v[wave];
  // wave w walks selection positions first, first + step, ... (one
  // workgroup: w, w + 8, ...; a pair: w + 8 half, w + 8 half + 16, ...)
  const int step = pair ? 2 * NW : NW;
  const int first = wave + (pair ? NW * pair->half : 0);
  const int nbw = cnt > first ? (cnt - first + step - 1) / step : 0;
  const int nent = item_entry_count<NW>(cnt);   // entries written by item_entries

  constexpr int PSH = kLo ? 9 : 5;   // page bits start here
  uint4 kr[NPF][NL], vr[NPF][NL];
  int ntok[NPF], lotok[NPF];
#pragma unroll
  for (int s = 0; s < NPF; ++s) {
    const int ie = first + step * s;
    const int e = ie < nent ? ent[ie] : -1;
    ntok[s] = e >= 0 ? (e & 31) : 0;
    lotok[s] = kLo && e >= 0 ? (e >> 5) & 15 : 0;
    const uint64_t off = (uint64_t)(uint32_t)(e >= 0 ? e >> PSH : 0) * pstride;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      kr[s][j] = ldg16_stream(kb + off + (size_t)j * ST::RPI * D);
      vr[s][j] = ldg16_stream(vb + off + (size_t)j * ST::RPI * D);
    }
    __builtin_amdgcn_sched_barrier(0);   // issue the slots in order (oldest = slot 0)
  }
  f32x4_t o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kNegInf, l = 0.0f;   // state of head `row` (meaningful in head lanes)

  for (int k0 = 0; k0 < nbw; k0 += NPF) {
#pragma unroll
    for (int s = 0; s < NPF; ++s) {
      const int k = k0 + s;
      // the block that refills this slot (entries past the written ones read as empty)
      const int ie = first + step * (k + NPF);
      const int en = ie < nent ? ent[ie] : -1;
      if (k < nbw) {
        // V rows past the block's tokens (a partly filled last page, or an
        // invalid entry) are zeroed: their weights are 0, but their contents
        // are unspecified and 0 * NaN would reach the output. K rows need no
        // such care: their logits are masked.
        if (ntok[s] < 16 || (kLo && lotok[s] > 0)) {
#pragma unroll
          for (int j = 0; j < NL; ++j) {
            const int tr = j * ST::RPI + lane / ST::LPR;
            if (tr >= ntok[s] || (kLo && tr < lotok[s])) vr[s][j] = make_uint4(0, 0, 0, 0);
          }
        }
        // stage the K and V tiles (row-major, padded rows)
        stage_k<D>(kt, kr[s], 0u);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          uint32_t* d = vt + (j * ST::RPI + lane / ST::LPR) * RW + 4 * (lane % ST::LPR);
          *reinterpret_cast<uint2*>(d) = make_uint2(vr[s][j].x, vr[s][j].y);
          *reinterpret_cast<uint2*>(d + 2) = make_uint2(vr[s][j].z, vr[s][j].w);
        }
        wave_lds_sync();
        // logits: lane holds head `row` for tokens 4kq + i
        f32x4_t z4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < KS; ++j) z4 = mfma_16x16x32(k_operand<D>(kt, j), qo.b[j], z4);
        float z[4], bm = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = head_lane && 4 * kq + i < ntok[s] && (!kLo || 4 * kq + i >= lotok[s]);
          z[i] = ok ? z4[i] * a.sm_scale_log2 : kNegInf;
          bm = fmaxf(bm, z[i]);
        }
        float lo, hi;
        xor_pair<16>(bm, lo, hi);
        bm = fmaxf(lo, hi);
        xor_pair<32>(bm, lo, hi);
        bm = fmaxf(lo, hi);
        const float mn = fmaxf(m, bm);
        // exp2 of values <= 0 with -inf -> 0 (mn = -inf: nothing seen yet, all 0)
        const float mref = mn == kNegInf ? 0.0f : mn;
        const float alpha = mn == kNegInf ? 1.0f : exp2_fast(m - mref);
        float p[4], ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = exp2_fast(z[i] - mref);
          ps += p[i];
        }
        xor_pair<16>(ps, lo, hi);
        ps = lo + hi;
        xor_pair<32>(ps, lo, hi);
        ps = lo + hi;
        l = l * alpha + ps;
        m = mn;
        // rescale o where a head's max grew (o rows = heads 0..3 in lanes 0..15)
        const float a0 = rl_f(alpha, 0), a1 = rl_f(alpha, 1), a2 = rl_f(alpha, 2),
                    a3 = rl_f(alpha, 3);
        if (a0 != 1.0f || a1 != 1.0f || a2 != 1.0f || a3 != 1.0f) {
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            o[n][0] *= a0; o[n][1] *= a1; o[n][2] *= a2; o[n][3] *= a3;
          }
        }
        // P in bf16 parts hi + lo (+ lo2 for fp32 output), in the A-operand
        // layout (row = head, k = 4 tokens)
        uint2 ph, pl, pm = make_uint2(0u, 0u);
        bf16x2_split(p[0], p[1], &ph.x);
        bf16x2_split(p[2], p[3], &ph.y);
        bf16x2_split(p[0], p[1], &pl.x);
        bf16x2_split(p[2], p[3], &pl.y);
        if (out32) pm = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        // o += P . V, one 16-dim tile at a time; B = V[tokens 4kq..+4][dim],
        // gathered by one transpose read: this lane addresses row
        // 4 kq + row / 4 at columns 4 (row % 4) of the 16-dim tile
        const uint16_t* vrow = reinterpret_cast<const uint16_t*>(vt) +
                               (4 * kq + (row >> 2)) * (2 * RW) + 4 * (row & 3);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint2 vb2 = lds_read_tr16(vrow + 16 * n);
          o[n] = mfma_16x16x16(ph, vb2, o[n]);
          o[n] = mfma_16x16x16(pl, vb2, o[n]);
          if (out32) o[n] = mfma_16x16x16(pm, vb2, o[n]);
        }
        wave_lds_sync();
      }
      __builtin_amdgcn_sched_barrier(0);   // refill after the use (loads complete in order)
      ntok[s] = en >= 0 ? (en & 31) : 0;
      lotok[s] = kLo && en >= 0 ? (en >> 5) & 15 : 0;
      const uint64_t off = (uint64_t)(uint32_t)(en >= 0 ? en >> PSH : 0) * pstride;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        kr[s][j] = ldg16_stream(kb + off + (size_t)j * ST::RPI * D);
        vr[s][j] = ldg16_stream(vb + off + (size_t)j * ST::RPI * D);
      }
    }
  }
  // wave states to LDS: o rows 0..3 (heads) live in lanes 0..15; the wave's
  // own K tile holds its o (its walk is over: every LDS read of the tile has
  // completed at the last wave_lds_sync)
  float* acc = sh.acc_of(wave);
  if (kq == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[h * D + 16 * n + row] = o[n][h];
    }
  }
  if (lane < 4) {
    sh.m[wave][lane] = m;
    sh.l[wave][lane] = l;
  }
  __syncthreads();
  // merge the wave states in wave order: output elements e = h * D + d,
  // EPT per thread
  constexpr int NTH = NW * kWave, EPT = (4 * D + NTH - 1) / NTH;
  float Mv[EPT], Ov[EPT], Lv[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + j * NTH;
    const int h = e / D;
    float M = kNegInf, O = 0.0f, Ls = 0.0f;
    if (e < 4 * D) {
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sh.m[w][h]);
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float f = exp2_fast(sh.m[w][h] - M);   // waves with m = -inf give 0
          O += f * sh.acc_of(w)[e];
          Ls += f * sh.l[w][h];
        }
      }
    }
    Mv[j] = M;
    Ov[j] = O;
    Lv[j] = Ls;
  }
  if (state) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      state->m[j] = Mv[j];
      state->o[j] = Ov[j];
      state->l[j] = Lv[j];
    }
    return;
  }
  if (split) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + j * NTH;
      const int h = e / D, d = e % D;
      if (e < 4 * D) {
        float* ph = split->part + (((size_t)r * a.num_q_heads + g * 4 + h) * split->num_splits +
                                   split->s) * (D + 2);
        store_split_word<kSplitStore>(ph + d, Ov[j]);
        if (d == 0) {
          store_split_word<kSplitStore>(ph + D, Mv[j]);
          store_split_word<kSplitStore>(ph + D + 1, Lv[j]);
        }
      }
    }
    return;
  }
  if constexpr (EPT == 1) {
    if (pair) {
      // publish, count the arrival, and let the second workgroup finish
      const int e = tid;
      const int h = e / D, d = e % D;
      float M = Mv[0], O = Ov[0], Ls = Lv[0];
      float* mine = pair->part + (size_t)pair->half * 4 * D;
      float* ml = pair->part + 2 * 4 * D;
      if (e < 4 * D) {
        st_dev(mine + e, O);
        if (d == 0) {
          st_dev(ml + pair->half * 8 + 2 * h, M);
          st_dev(ml + pair->half * 8 + 2 * h + 1, Ls);
        }
      }
      wait_stores();
      __syncthreads();
      if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(pair->arrivals, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        sh.m[0][0] = __int_as_float(prev == 1u ? 1 : 0);
      }
      __syncthreads();
      if (__float_as_int(sh.m[0][0]) == 0) return;   // the other workgroup finishes
      if (e < 4 * D) {
        const int oh = 1 - pair->half;
        const float Mo = ld_dev(ml + oh * 8 + 2 * h), Lo = ld_dev(ml + oh * 8 + 2 * h + 1);
        const float Oo = ld_dev(pair->part + (size_t)oh * 4 * D + e);
        // merge in half order (half 0 first), so the result does not depend on
        // which workgroup arrives last
        const float M0 = pair->half == 0 ? M : Mo, M1 = pair->half == 0 ? Mo : M;
        const float O0 = pair->half == 0 ? O : Oo, O1 = pair->half == 0 ? Oo : O;
        const float L0 = pair->half == 0 ? Ls : Lo, L1 = pair->half == 0 ? Lo : Ls;
        const float Mn = fmaxf(M0, M1);
        O = 0.0f;
        Ls = 0.0f;
        if (Mn != kNegInf) {
          const float f0 = exp2_fast(M0 - Mn), f1 = exp2_fast(M1 - Mn);
          O = f0 * O0 + f1 * O1;
          Ls = f0 * L0 + f1 * L1;
        }
        M = Mn;
      }
      Mv[0] = M;
      Ov[0] = O;
      Lv[0] = Ls;
    }
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + j * NTH;
    const int h = e / D, d = e % D;
    if (e < 4 * D) {
      const float M = Mv[j], Ls = Lv[j];
      const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
      const size_t idx = ((size_t)r * a.num_q_heads + g * 4 + h) * D + d;
      if (out32) reinterpret_cast<float*>(a.out)[idx] = Ov[j] * inv;
      else reinterpret_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_rne(Ov[j] * inv);
      if (a.lse && d == 0)
        a.lse[(size_t)r * a.num_q_heads + g * 4 + h] =
            (M == kNegInf || !(Ls > 0.0f)) ? kNegInf : (M + log2f(Ls)) * kLn2;
    }
  }
}

}  // namespace ls

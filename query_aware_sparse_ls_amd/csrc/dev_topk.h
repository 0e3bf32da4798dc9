// Per (request, KV head) top-k over block scores plus forced sink / recent
// blocks, emitted in ascending block order -- one workgroup of 256 or 1024
// threads (device code shared by the standalone top-k kernel and the
// per-(request, kv head) selection and decode-step kernels).
//
// Vortex post: I = top-k_j(s_j) ("Why Long Generations Are Expensive"). The
// post notes that radix top-k, which buckets values by their digits, slows
// down when many high scores share a bucket, and that a monotonic remapping
// of the scores spreads them over the buckets ("Making it fast"). This code
// keeps the exact answer and uses that idea for speed: each pass buckets the
// undecided candidates by a monotone linear map of the score onto 256 buckets
// between their min and max (fp32 subtraction and multiplication by a
// positive constant are monotone), takes every candidate above the bucket
// holding the k-th score, drops those below, and refines the boundary bucket.
// Once at most 64 candidates remain undecided, each of them is ranked by
// counting the undecided candidates ahead of it in the order (score
// descending, block index ascending), and the first ones are taken: ties go
// to the lowest block index and the result is unique and deterministic.
// Equal or pathological scores fall back to a bitwise threshold search on an
// order-preserving integer key followed by a lowest-index fill.
//
// Thread t holds the scores of candidates [t*PER, t*PER + PER) in registers,
// so index order is thread order, then register order, and ordered counts are
// one workgroup prefix sum.
#pragma once

#include "ls_internal.h"

namespace ls {

constexpr int kTopkThreads = 256;     // workgroup size of the standalone top-k kernel
constexpr int kTopkMaxIters = 24;
constexpr int kTopkMaxCand = 16384;
constexpr int kTopkMaxWaves = 16;     // workgroups of up to 1024 threads

struct TopkLds {
  int hist[256];
  float red_f[2][kTopkMaxWaves];
  int red_i[4][kTopkMaxWaves];
  int bstar, cabove, cstar;   // boundary bucket, candidates above it, candidates in it
  float list_key[kWave];   // the last (at most 64) undecided candidates, in any order
  int list_idx[kWave];
  int list_n;
};

// Monotone bucket of a score between mn and mx (scale = 256 / (mx - mn)).
__device__ __forceinline__ int bucket_of(float key, float mn, float scale) {
  const int b = (int)((key - mn) * scale);
  return b > 255 ? 255 : (b < 0 ? 0 : b);
}

// Workgroup total of a small per-thread count (< 128) over NW waves; one
// barrier.
template <int NW>
__device__ __forceinline__ int wg_sum_i(TopkLds& sh, int v, int slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int tot;
  (void)wave_excl_scan_small<7>(v, &tot);
  if (lane == 0) sh.red_i[slot][wave] = tot;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += sh.red_i[slot][w];
  return s;
}

// Exclusive prefix sum of a small per-thread count (< 128) over the NW waves
// of the workgroup in thread order; *total = sum. One barrier.
template <int NW>
__device__ __forceinline__ int wg_excl_scan_i(TopkLds& sh, int v, int slot, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int wtot;
  const int pre = wave_excl_scan_small<7>(v, &wtot);
  if (lane == 0) sh.red_i[slot][wave] = wtot;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = sh.red_i[slot][w];
    before += (w < wave) ? x : 0;
    tot += x;
  }
  *total = tot;
  return before + pre;
}

// (a before b) in the selection order: higher score first, then lower index.
__device__ __forceinline__ bool ahead(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Inclusive suffix sum over the wave (lane l gets the sum of lanes >= l) of
// per-lane bucket counts (< 2^15), by bit planes.
__device__ __forceinline__ int tot_minus_prefix(int v, int* total) {
  const int pre = wave_excl_scan_small<15>(v, total);
  return *total - pre;
}

// range (optional, LDS): the candidates' smallest scores in range[0 ..
// range_n) and largest in range[range_n .. 2 range_n), when the producer of
// the scores found them; the first pass then needs no reduction.
// kPad16: srow holds candidate e at srow[e + e / 16] (one pad word after
// every 16, so that the thread-owns-PER-consecutive reads of an LDS row hit
// distinct banks).
// srow: scores of candidate blocks c0 .. c1-1 (srow[0] is block c0), in
// global memory or LDS; c1 - c0 <= NT * PER <= kTopkMaxCand. Called by all
// NT threads of the workgroup. The selection goes to out[0 .. max_selected)
// (unused entries -1) and its size to *count_out; sel_lds, when given, gets a
// copy of the first min(total, max_selected) entries. Returns that count.
// kDev: out and *count_out are written with device-coherent stores, for
// readers in other workgroups of the same launch.
template <int PER, int NT = kTopkThreads, bool kPad16 = false, bool kDev = false>
__device__ int topk_wg(const float* __restrict__ srow, const ReqGeom& geo, int k,
                        int32_t* __restrict__ out, int max_selected,
                        int32_t* __restrict__ count_out, TopkLds& sh,
                        int32_t* __restrict__ sel_lds = nullptr,
                        const float* __restrict__ range = nullptr, int range_n = 0) {
  constexpr int NW = NT / kWave;
  static_assert(NT % kWave == 0 && NW <= kTopkMaxWaves && NT >= 256, "workgroup size");
  static_assert(PER >= 1 && PER <= 64 && PER * NT <= kTopkMaxCand, "PER");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = geo.c1 - geo.c0;
  int need = k < n ? k : n;
  if (tid == 0) sh.list_n = 0;   // first used after at least one barrier
  float key[PER];
  unsigned long long act = 0, sel = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    key[j] = e < n ? srow[kPad16 ? e + (e >> 4) : e] : 0.0f;
    act |= (unsigned long long)(e < n) << j;
  }
  if (need >= n) {
    sel = act;
    act = 0;
    need = 0;
  }
  bool robust = false;
  int known = -1;   // the undecided count, when the last pass's histogram gives it
  for (int it = 0; need > 0; ++it) {
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    int cnt;
    if (known >= 0 && (known <= need || known <= kWave)) {
      cnt = known;   // the remainder is filled or sorted: no range needed
    } else if (it == 0 && range && n > kWave) {   // (a barrier precedes any ranking)
      cnt = n;       // every candidate, over the range the scores' producer found
      for (int w = 0; w < range_n; ++w) {
        mn = fminf(mn, range[w]);
        mx = fmaxf(mx, range[range_n + w]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const bool a = (act >> j) & 1ull;
        mn = a ? fminf(mn, key[j]) : mn;
        mx = a ? fmaxf(mx, key[j]) : mx;
      }
      (void)wave_excl_scan_small<7>(__popcll(act), &cnt);
      mn = wave_min_fast(mn);
      mx = wave_max_fast(mx);
      if (lane == 0) { sh.red_i[0][wave] = cnt; sh.red_f[0][wave] = mn; sh.red_f[1][wave] = mx; }
      __syncthreads();
      cnt = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        cnt += sh.red_i[0][w];
        mn = fminf(mn, sh.red_f[0][w]);
        mx = fmaxf(mx, sh.red_f[1][w]);
      }
      __syncthreads();
    }
    if (cnt <= need) {          // the boundary bucket holds exactly the remainder
      sel |= act;
      act = 0;
      break;
    }
    if (cnt <= kWave) {
      // the undecided candidates (at most one wave's worth) go to a list in
      // thread order; wave 0 ranks them, lane i entry i, by counting the
      // entries ahead of it (read from the other lanes; the order is total),
      // flags the first `need`, and the owners take the flagged ones
      int listed;
      const int base = wg_excl_scan_i<NW>(sh, __popcll(act), 1, &listed);
      listed = listed < kWave ? listed : kWave;
      {
        int pos = base;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          if ((act >> j) & 1ull) {
            if (pos < kWave) {
              sh.list_key[pos] = key[j];
              sh.list_idx[pos] = tid * PER + j;
            }
            ++pos;
          }
        }
      }
      __syncthreads();
      if (tid < kWave) {
        const float mk = lane < listed ? sh.list_key[lane] : 0.0f;
        const int mi = lane < listed ? sh.list_idx[lane] : 0;
        int rank = 0;
        for (int u = 0; u < listed; ++u)
          rank += ahead(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), u)),
                        __builtin_amdgcn_readlane(mi, u), mk, mi);
        if (lane < listed) sh.list_idx[lane] = rank < need ? 1 : 0;
      }
      __syncthreads();
      {
        int pos = base;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          if ((act >> j) & 1ull) {
            if (pos < kWave && sh.list_idx[pos]) sel |= 1ull << j;
            ++pos;
          }
        }
      }
      act = 0;
      break;
    }
    const float range = mx - mn;
    const float scale = 256.0f / range;
    if (!(range > 0.0f) || !(scale < __builtin_huge_valf()) || it >= kTopkMaxIters) {
      robust = true;
      break;
    }
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((act >> j) & 1ull) atomicAdd(&sh.hist[bucket_of(key[j], mn, scale)], 1);
    __syncthreads();
    if (wave == 0) {
      // suffix counts over the 256 buckets, 4 per lane
      const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
      const int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
      // suffix sums of the lane totals: total - exclusive prefix
      int tot;
      const int lsum = h0 + h1 + h2 + h3;
      const int suf = tot_minus_prefix(lsum, &tot);
      const int s3 = suf - h0 - h1 - h2, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
      int best = -1, sbest = 0, hbest = 0;
      if (s0 >= need) { best = 4 * lane; sbest = s0; hbest = h0; }
      if (s1 >= need) { best = 4 * lane + 1; sbest = s1; hbest = h1; }
      if (s2 >= need) { best = 4 * lane + 2; sbest = s2; hbest = h2; }
      if (s3 >= need) { best = 4 * lane + 3; sbest = s3; hbest = h3; }
      const int bmax = (int)wave_max_fast((float)best);
      if (best == bmax && best >= 0) {
        sh.bstar = best;
        sh.cabove = sbest - hbest;
        sh.cstar = hbest;
      }
    }
    __syncthreads();
    const int bstar = sh.bstar, cabove = sh.cabove;
    known = sh.cstar;
    unsigned long long up = 0, keep = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int b = bucket_of(key[j], mn, scale);
      up |= (unsigned long long)(b > bstar) << j;
      keep |= (unsigned long long)(b == bstar) << j;
    }
    sel |= act & up;
    act &= keep;
    need -= cabove;
    __syncthreads();
  }

  if (robust) {
    // need-th largest order-preserving key among the undecided, bit by bit
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int c = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) c += ((act >> j) & 1ull) && score_key(key[j]) >= cand;
      c = wg_sum_i<NW>(sh, c, 2 + (bit & 1));   // alternating slots: one barrier per bit
      if (c >= need) prefix = cand;
    }
    unsigned long long above = 0, equal = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t uk = score_key(key[j]);
      above |= (unsigned long long)(uk > prefix) << j;
      equal |= (unsigned long long)(uk == prefix) << j;
    }
    above &= act;
    equal &= act;
    __syncthreads();
    const int nabove = wg_sum_i<NW>(sh, __popcll(above), 0);
    __syncthreads();
    int tot;
    int pos = wg_excl_scan_i<NW>(sh, __popcll(equal), 1, &tot);
    const int fill = need - nabove;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((equal >> j) & 1ull) {
        if (pos < fill) sel |= 1ull << j;
        ++pos;
      }
    }
    sel |= above;
    __syncthreads();
  }

  // emit: forced [0, c0), the chosen candidates in order, forced [c1, nb)
  int ncand;
  int pos = geo.c0 + wg_excl_scan_i<NW>(sh, __popcll(sel), 2, &ncand);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if ((sel >> j) & 1ull) {
      if (pos < max_selected) {
        const int b = geo.c0 + tid * PER + j;
        st_x<kDev>(&out[pos], b);
        if (sel_lds) sel_lds[pos] = b;
      }
      ++pos;
    }
  }
  const int nlow = geo.c0, nhigh = geo.nb - geo.c1;
  const int total = nlow + ncand + nhigh;
  for (int i = tid; i < nlow; i += NT) {
    if (i < max_selected) {
      st_x<kDev>(&out[i], i);
      if (sel_lds) sel_lds[i] = i;
    }
  }
  for (int i = tid; i < nhigh; i += NT) {
    const int p = nlow + ncand + i;
    if (p < max_selected) {
      st_x<kDev>(&out[p], geo.c1 + i);
      if (sel_lds) sel_lds[p] = geo.c1 + i;
    }
  }
  for (int i = total + tid; i < max_selected; i += NT) st_x<kDev>(&out[i], -1);
  const int stored = total < max_selected ? total : max_selected;
  if (tid == 0) st_x<kDev>(count_out, stored);
  __syncthreads();
  return stored;
}

// ---------------------------------------------------------------------------
// topk_fast: the same exact selection (the first k candidates under (score
// descending, block index ascending), forced blocks added, ascending
// output) for up to kTopkFastMaxBlocks blocks when the candidates' score
// range is known up front, with fewer barriers than topk_wg:
//  * each bucketing pass has its own pre-zeroed histogram (no zeroing
//    barrier), and every wave finds the boundary bucket by itself from a DPP
//    prefix sum over the 256 buckets (no second barrier);
//  * the kept blocks (candidates and forced) go into an LDS bitmap, from
//    which one wave writes the ascending selection (one word per lane, a
//    wave prefix sum of the word counts gives each lane its output slot).
// Degenerate score ranges, or more passes than histograms, fall back to
// topk_wg on the same scores (same result).
constexpr int kTopkFastPasses = 4;
constexpr int kTopkFastMaxBlocks = 4096;

template <int MAXB = kTopkFastMaxBlocks>
struct TopkFastLds {
  static_assert(MAXB % 32 == 0, "whole bitmap words");
  int hist[kTopkFastPasses][256];
  unsigned bm[MAXB / 32];
  float list_key[kWave];
  int list_idx[kWave];
  int list_n;
  int total;
};

// Inclusive prefix sum over the 64 lanes: DPP shifts inside each 16-lane
// row, then the row totals read into scalars.
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = __lane_id() >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// topk_wg on a padded LDS score row, as a real call: the fast path's rare
// fallback should not add its registers to the caller's.
template <int PER, int NT, bool kDev>
__device__ __noinline__ int topk_fallback(const float* srow, const ReqGeom& geo, int k,
                                          int32_t* out, int max_selected, int32_t* count_out,
                                          TopkLds& sh, int32_t* sel_lds) {
  return topk_wg<PER, NT, true, kDev>(srow, geo, k, out, max_selected, count_out, sh, sel_lds);
}

// srow: LDS, candidate e at srow[e + e / 16] (c1 - c0 <= NT * PER); mn0 / mx0:
// the smallest and largest candidate score. Called by all NT threads; the
// caller synchronises after writing srow. The selection is handed out as
// emit(p, b) for every output position p < max_selected: b = the p-th
// selected block in ascending order, or -1 past the selection (wave 0
// calls it, except on the fallback path, where every thread may; the
// fallback writes the selection to fb_out with device-coherent stores and
// reads it back). Returns the stored count, min(selected, max_selected).
// MAXB: the bitmap's blocks (geo.nb <= MAXB).
template <int PER, int NT, class Emit, int MAXB>
__device__ int topk_fast(const float* __restrict__ srow, const ReqGeom& geo, int k,
                         int max_selected, TopkFastLds<MAXB>& sh, TopkLds& fallback,
                         int32_t* __restrict__ fb_out, int32_t* __restrict__ fb_count, float mn0,
                         float mx0, Emit emit) {
  constexpr int NW = NT / kWave;
  static_assert(NT % kWave == 0 && NW <= kTopkMaxWaves && PER >= 1 && PER <= 32, "shape");
  static_assert(NT * PER <= MAXB, "blocks");
  constexpr int WPL = (MAXB / 32 + kWave - 1) / kWave;   // bitmap words per lane
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = geo.c1 - geo.c0;
  for (int i = tid; i < kTopkFastPasses * 256; i += NT) (&sh.hist[0][0])[i] = 0;
  for (int i = tid; i < MAXB / 32; i += NT) sh.bm[i] = 0u;
  if (tid == 0) sh.list_n = 0;
  float key[PER];
  uint32_t act = 0, sel = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    key[j] = e < n ? srow[e + (e >> 4)] : 0.0f;
    act |= (uint32_t)(e < n) << j;
  }
  int need = k < n ? k : n;
  int cnt = n;   // undecided candidates (exact: from the last pass's histogram)
  float mn = mn0, mx = mx0;
  bool robust = false;
  __syncthreads();
  for (int it = 0; need > 0; ++it) {
    if (cnt <= need) {   // every undecided candidate is in
      sel |= act;
      act = 0;
      break;
    }
    if (cnt <= kWave) {
      // list the undecided (at most one wave's worth); wave 0 ranks them,
      // lane i entry i, by counting the entries ahead of it (read from the
      // other lanes), and the first `need` go straight into the bitmap
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if ((act >> j) & 1u) {
          const int pos = atomicAdd(&sh.list_n, 1);
          sh.list_key[pos] = key[j];
          sh.list_idx[pos] = tid * PER + j;
        }
      }
      __syncthreads();
      if (tid < kWave) {
        const float mk = lane < cnt ? sh.list_key[lane] : 0.0f;
        const int mi = lane < cnt ? sh.list_idx[lane] : 0;
        int rank = 0;
        for (int u = 0; u < cnt; ++u)
          rank += ahead(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), u)),
                        __builtin_amdgcn_readlane(mi, u), mk, mi);
        if (lane < cnt && rank < need) {
          const int b = geo.c0 + mi;
          atomicOr(&sh.bm[b >> 5], 1u << (b & 31));
        }
      }
      act = 0;
      break;
    }
    const float range = mx - mn;
    const float scale = 256.0f / range;
    if (it >= kTopkFastPasses || !(range > 0.0f) || !(scale < __builtin_huge_valf())) {
      robust = true;
      break;
    }
    int* h = sh.hist[it];
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((act >> j) & 1u) atomicAdd(&h[bucket_of(key[j], mn, scale)], 1);
    __syncthreads();
    // every wave: the boundary bucket b* = the highest bucket whose suffix
    // count (candidates in buckets >= b) is at least `need`
    const int h0 = h[4 * lane], h1 = h[4 * lane + 1], h2 = h[4 * lane + 2], h3 = h[4 * lane + 3];
    const int lsum = (h0 + h1) + (h2 + h3);
    const int incl = wave_incl_scan_dpp(lsum);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int s0 = total - (incl - lsum), s1 = s0 - h0, s2 = s1 - h1, s3 = s2 - h2;
    int best = -1, sb = 0, hb = 0;
    if (s0 >= need) { best = 4 * lane; sb = s0; hb = h0; }
    if (s1 >= need) { best = 4 * lane + 1; sb = s1; hb = h1; }
    if (s2 >= need) { best = 4 * lane + 2; sb = s2; hb = h2; }
    if (s3 >= need) { best = 4 * lane + 3; sb = s3; hb = h3; }
    const unsigned long long m = __ballot(best >= 0);   // lane 0 is in: s0 = cnt >= need
    const int L = 63 - __builtin_clzll(m);
    const int bstar = __builtin_amdgcn_readlane(best, L);
    const int cabove = __builtin_amdgcn_readlane(sb, L) - __builtin_amdgcn_readlane(hb, L);
    const int cstar = __builtin_amdgcn_readlane(hb, L);
    uint32_t up = 0, keep = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int b = bucket_of(key[j], mn, scale);
      up |= (uint32_t)(b > bstar) << j;
      keep |= (uint32_t)(b == bstar) << j;
    }
    sel |= act & up;
    act &= keep;
    need -= cabove;
    cnt = cstar;
    // the boundary bucket's score interval (the map stays monotone if it is
    // not exact: keys outside clamp to the edge buckets)
    const float lo = mn + (float)bstar / scale, hi = mn + (float)(bstar + 1) / scale;
    mn = lo;
    mx = hi;
  }
  if (robust) {
    const int stored = topk_fallback<PER, NT, true>(srow, geo, k, fb_out, max_selected,
                                                    fb_count, fallback, nullptr);
    wait_stores();
    __syncthreads();
    for (int p = tid; p < max_selected; p += NT) emit(p, ld_dev(&fb_out[p]));
    __syncthreads();
    return stored;
  }
  // the kept blocks into the bitmap: this thread's candidates (consecutive
  // blocks), then the forced ones
  {
    int word = -1;
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((sel >> j) & 1u) {
        const int b = geo.c0 + tid * PER + j;
        if ((b >> 5) != word) {
          if (bits) atomicOr(&sh.bm[word], bits);
          word = b >> 5;
          bits = 0;
        }
        bits |= 1u << (b & 31);
      }
    }
    if (bits) atomicOr(&sh.bm[word], bits);
  }
  for (int i = tid; i < geo.c0; i += NT) atomicOr(&sh.bm[i >> 5], 1u << (i & 31));
  for (int i = geo.c1 + tid; i < geo.nb; i += NT) atomicOr(&sh.bm[i >> 5], 1u << (i & 31));
  __syncthreads();
  if (tid < kWave) {
    const int nwords = (geo.nb + 31) >> 5;
    uint32_t w[WPL];
    int pos[WPL];
    int base = 0;
#pragma unroll
    for (int q = 0; q < WPL; ++q) {
      const int wi = q * kWave + lane;
      w[q] = wi < nwords ? sh.bm[wi] : 0u;
      const int c = __popc(w[q]);
      const int incl = wave_incl_scan_dpp(c);
      pos[q] = base + incl - c;
      base += __builtin_amdgcn_readlane(incl, 63);
    }
    const int total = base;
#pragma unroll
    for (int q = 0; q < WPL; ++q) {
      uint32_t x = w[q];
      int p = pos[q];
      while (x) {
        const int b = (q * kWave + lane) * 32 + (__ffs(x) - 1);
        x &= x - 1;
        if (p < max_selected) emit(p, b);
        ++p;
      }
    }
    for (int i = total + lane; i < max_selected; i += kWave) emit(i, -1);
    if (lane == 0) sh.total = total < max_selected ? total : max_selected;
  }
  __syncthreads();
  return sh.total;
}

__device__ __forceinline__ int topk_budget(const TopkArgs& a, const ReqGeom& geo) {
  int k = a.topk;
  if (k < 0) {
    const int nforced = geo.nb - (geo.c1 - geo.c0);
    const int total = (int)ceilf(a.keep_ratio * (float)geo.nb);
    k = (total > nforced ? total : nforced) - nforced;
  }
  return k;
}

}  // namespace ls

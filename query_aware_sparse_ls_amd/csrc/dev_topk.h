// Per (request, KV head) top-k over block scores plus forced sink / recent
// blocks, emitted in ascending block order -- one wavefront, no workgroup
// barriers (wave-level device code shared by the standalone top-k kernel and
// the fused decode-step kernel).
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
// Once at most 64 candidates remain undecided they are ranked exactly, one
// per lane, by (score descending, block index ascending): ties go to the
// lowest block index and the result is unique and deterministic. Equal or
// pathological scores fall back to a bitwise threshold search on an
// order-preserving integer key followed by a lowest-index fill.
//
// The wave's candidate scores live in LDS; element e (block c0 + e) is
// handled by lane e % 64 as bit e / 64 of that lane's 64-bit masks, so index
// order is (bit, lane) order and every ordered count is a wave ballot.
#pragma once

#include "ls_internal.h"

namespace ls {

constexpr int kTopkMaxIters = 24;

// MAXC: candidate capacity (a multiple of 64, at most 4096).
template <int MAXC>
struct WaveTopkLds {
  static_assert(MAXC % kWave == 0 && MAXC <= 64 * kWave, "capacity");
  float keys[MAXC];
  int hist[256];
  float list_key[kWave];
  int list_idx[kWave];
  unsigned long long mark[kWave];
};

// Monotone bucket of a score between mn and mx (scale = 256 / (mx - mn)).
__device__ __forceinline__ int bucket_of(float key, float mn, float scale) {
  const int b = (int)((key - mn) * scale);
  return b > 255 ? 255 : (b < 0 ? 0 : b);
}

__device__ __forceinline__ int lanes_below(unsigned long long m, int lane) {
  return __popcll(m & ((1ull << lane) - 1ull));
}

// The `need` lowest-index members of `pool` (bit j of lane l = element 64j + l).
__device__ __forceinline__ unsigned long long lowest_fill(unsigned long long pool, int need,
                                                          int nbits, int lane) {
  unsigned long long take = 0;
  int base = 0;
  for (int j = 0; j < nbits && base < need; ++j) {
    const bool b = (pool >> j) & 1ull;
    const unsigned long long m = __ballot(b);
    if (b && base + lanes_below(m, lane) < need) take |= 1ull << j;
    base += __popcll(m);
  }
  return take;
}

// srow: scores of candidate blocks c0 .. c1-1 (srow[0] is block c0);
// c1 - c0 <= MAXC.
template <int MAXC>
__device__ void topk_wave(const float* __restrict__ srow, const ReqGeom& geo, int k,
                          int32_t* __restrict__ out, int max_selected,
                          int32_t* __restrict__ count_out, WaveTopkLds<MAXC>& sh, int lane) {
  const int n = geo.c1 - geo.c0;
  const int nbits = (n + kWave - 1) / kWave;
  int need = k < n ? k : n;
  unsigned long long act = 0, sel = 0;
  for (int j0 = 0; j0 < nbits; j0 += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = (j0 + u) * kWave + lane;
      t[u] = (j0 + u < nbits && e < n) ? srow[e] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = (j0 + u) * kWave + lane;
      if (j0 + u < nbits && e < n) {
        sh.keys[e] = t[u];
        act |= 1ull << (j0 + u);
      }
    }
  }
  wave_lds_sync();
  if (need >= n) {
    sel = act;
    act = 0;
    need = 0;
  }
  bool robust = false;
  for (int it = 0; need > 0; ++it) {
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    for (int j = 0; j < nbits; ++j) {
      if ((act >> j) & 1ull) {
        const float x = sh.keys[j * kWave + lane];
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
    }
    const int cnt = wave_sum(__popcll(act));
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (cnt <= need) {          // the boundary bucket holds exactly the remainder
      sel |= act;
      act = 0;
      break;
    }
    if (cnt <= kWave) {
      // exact ranking of the undecided candidates, one per lane
      int pos = wave_excl_scan(__popcll(act), lane);
      for (int j = 0; j < nbits; ++j) {
        if ((act >> j) & 1ull) {
          const int e = j * kWave + lane;
          sh.list_key[pos] = sh.keys[e];
          sh.list_idx[pos] = e;
          ++pos;
        }
      }
      sh.mark[lane] = 0ull;
      wave_lds_sync();
      if (lane < cnt) {
        const float mk = sh.list_key[lane];
        const int mi = sh.list_idx[lane];
        int rank = 0;
        for (int u = 0; u < cnt; ++u) {
          const float ok = sh.list_key[u];
          const int oi = sh.list_idx[u];
          rank += (ok > mk) || (ok == mk && oi < mi);
        }
        if (rank < need) atomicOr(&sh.mark[mi % kWave], 1ull << (mi / kWave));
      }
      wave_lds_sync();
      sel |= sh.mark[lane];
      act = 0;
      break;
    }
    const float range = mx - mn;
    const float scale = 256.0f / range;
    if (!(range > 0.0f) || !(scale < __builtin_huge_valf()) || it >= kTopkMaxIters) {
      robust = true;
      break;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.hist[lane * 4 + i] = 0;
    wave_lds_sync();
    for (int j = 0; j < nbits; ++j) {
      if ((act >> j) & 1ull)
        atomicAdd(&sh.hist[bucket_of(sh.keys[j * kWave + lane], mn, scale)], 1);
    }
    wave_lds_sync();
    // suffix counts over 256 buckets, 4 per lane
    const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
    const int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
    int suf = h0 + h1 + h2 + h3;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int nx = __shfl_down(suf, o, kWave);
      if (lane + o < kWave) suf += nx;
    }
    const int s3 = suf - h0 - h1 - h2, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
    int best = -1, sbest = 0, hbest = 0;
    if (s0 >= need) { best = 4 * lane; sbest = s0; hbest = h0; }
    if (s1 >= need) { best = 4 * lane + 1; sbest = s1; hbest = h1; }
    if (s2 >= need) { best = 4 * lane + 2; sbest = s2; hbest = h2; }
    if (s3 >= need) { best = 4 * lane + 3; sbest = s3; hbest = h3; }
    int bstar = best;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) bstar = max(bstar, __shfl_xor(bstar, o, kWave));
    // count above the boundary bucket, from the lane that owns it
    const int cabove = __shfl(sbest - hbest, bstar >> 2, kWave);
    for (int j = 0; j < nbits; ++j) {
      if ((act >> j) & 1ull) {
        const int b = bucket_of(sh.keys[j * kWave + lane], mn, scale);
        if (b > bstar) { sel |= 1ull << j; act &= ~(1ull << j); }
        else if (b < bstar) { act &= ~(1ull << j); }
      }
    }
    need -= cabove;
    wave_lds_sync();
  }

  if (robust) {
    // need-th largest order-preserving key among the undecided, bit by bit
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int c = 0;
      for (int j = 0; j < nbits; ++j)
        c += ((act >> j) & 1ull) && score_key(sh.keys[j * kWave + lane]) >= cand;
      if (wave_sum(c) >= need) prefix = cand;
    }
    unsigned long long above = 0, equal = 0;
    for (int j = 0; j < nbits; ++j) {
      if ((act >> j) & 1ull) {
        const uint32_t uk = score_key(sh.keys[j * kWave + lane]);
        if (uk > prefix) above |= 1ull << j;
        else if (uk == prefix) equal |= 1ull << j;
      }
    }
    const int nabove = wave_sum(__popcll(above));
    sel |= above | lowest_fill(equal, need - nabove, nbits, lane);
  }

  // emit: forced [0, c0), the chosen candidates, forced [c1, nb), ascending
  const int nlow = geo.c0, nhigh = geo.nb - geo.c1;
  int pos = nlow;
  for (int j = 0; j < nbits; ++j) {
    const bool b = (sel >> j) & 1ull;
    const unsigned long long m = __ballot(b);
    const int p = pos + lanes_below(m, lane);
    if (b && p < max_selected) out[p] = geo.c0 + j * kWave + lane;
    pos += __popcll(m);
  }
  const int ncand = pos - nlow;
  const int total = nlow + ncand + nhigh;
  for (int i = lane; i < nlow; i += kWave)
    if (i < max_selected) out[i] = i;
  for (int i = lane; i < nhigh; i += kWave)
    if (nlow + ncand + i < max_selected) out[nlow + ncand + i] = geo.c1 + i;
  for (int i = total + lane; i < max_selected; i += kWave) out[i] = -1;
  if (lane == 0) *count_out = total < max_selected ? total : max_selected;
  wave_lds_sync();
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

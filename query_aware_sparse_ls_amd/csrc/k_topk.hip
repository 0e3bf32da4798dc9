// Per (request, KV head) top-k over block scores, plus forced sink / recent
// blocks, emitted in ascending block order.
//
// Vortex post: I = top-k_j(s_j) ("Why Long Generations Are Expensive"); the
// standard radix top-k "repeatedly buckets values by their digits" and
// degrades when many high scores share a bucket, which the post counters with
// a monotonic remapping of the scores ("Making it fast"). This kernel keeps
// the exact result and uses that idea for speed: each pass buckets the still
// undecided candidates by a monotone linear map of their score onto 256
// buckets between the current min and max (monotone because fp32 subtraction
// and multiplication by a positive constant are monotone), so scores spread
// over the buckets instead of piling into the few buckets their exponent bits
// would give. Candidates above the bucket that holds the k-th score are
// taken, those below are dropped, and the boundary bucket is refined. Once at
// most 256 candidates remain undecided, each is ranked exactly against the
// others by (score descending, block index ascending), so ties go to the
// lowest block index and the result is unique and deterministic. Equal-score
// or pathological inputs fall back to a bitwise threshold search on an
// order-preserving integer key plus a lowest-index fill.
//
// One workgroup of 256 threads per (request, KV head); thread t holds the
// scores of candidates [t*PER, t*PER + PER) in registers, so index order is
// thread order, then register order.
#include "dev_topk.h"

namespace ls {

constexpr int kTopkThreads = 256;

struct TopkShared {
  int hist[256];
  float rf[3][4];
  int ri[4][4];
  int bstar, cabove;
  int list_n;
  float list_key[kTopkThreads];
  int list_idx[kTopkThreads];
  uint32_t bitmap[16384 / 32];
};

// Workgroup reductions: (count, min, max) in one round trip through LDS.
__device__ __forceinline__ void wg_cnt_min_max(TopkShared& sh, int& cnt, float& mn, float& mx) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  cnt = wave_sum(cnt);
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) { sh.ri[0][wave] = cnt; sh.rf[0][wave] = mn; sh.rf[1][wave] = mx; }
  __syncthreads();
  cnt = sh.ri[0][0] + sh.ri[0][1] + sh.ri[0][2] + sh.ri[0][3];
  mn = fminf(fminf(sh.rf[0][0], sh.rf[0][1]), fminf(sh.rf[0][2], sh.rf[0][3]));
  mx = fmaxf(fmaxf(sh.rf[1][0], sh.rf[1][1]), fmaxf(sh.rf[1][2], sh.rf[1][3]));
  __syncthreads();
}

__device__ __forceinline__ int wg_sum(TopkShared& sh, int v, int slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = wave_sum(v);
  if (lane == 0) sh.ri[slot][wave] = v;
  __syncthreads();
  v = sh.ri[slot][0] + sh.ri[slot][1] + sh.ri[slot][2] + sh.ri[slot][3];
  __syncthreads();
  return v;
}

// Exclusive prefix sum over the workgroup (thread order).
__device__ __forceinline__ int wg_excl_scan(TopkShared& sh, int v, int slot, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(v, lane);
  if (lane == 63) sh.ri[slot][wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = sh.ri[slot][w];
    before += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

template <int PER>
__device__ __forceinline__ uint64_t lowest_index_fill(TopkShared& sh, uint64_t pool, int need) {
  // take the `need` lowest-index members of `pool` (index order = thread, register)
  int mine = __popcll(pool), total;
  const int before = wg_excl_scan(sh, mine, 2, &total);
  uint64_t take = 0;
  int pos = before;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if ((pool >> j) & 1ull) {
      if (pos < need) take |= 1ull << j;
      ++pos;
    }
  }
  return take;
}

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void topk_wg_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int g = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
  const int ncand = geo.c1 - geo.c0;
  const int nforced = geo.nb - ncand;
  (void)nforced;
  const int k = topk_budget(a, geo);
  int need = k < ncand ? k : ncand;

  const float* srow = a.scores + ((size_t)r * a.num_kv_heads + g) * a.b.max_blocks + geo.c0;
  float key[PER];
  uint64_t act = 0, sel = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    key[j] = 0.0f;
    if (e < ncand) {
      key[j] = srow[e];
      act |= 1ull << j;
    }
  }
  const int nwords = (geo.nb + 31) >> 5;
  for (int w = tid; w < nwords; w += kTopkThreads) sh.bitmap[w] = 0u;
  if (tid == 0) sh.list_n = 0;
  __syncthreads();

  if (need >= ncand) {
    sel = act;
    act = 0;
    need = 0;
  }
  bool robust = false;
  for (int it = 0; need > 0; ++it) {
    int cnt = __popcll(act);
    float mn = __int_as_float(0x7f800000), mx = -__int_as_float(0x7f800000);
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((act >> j) & 1ull) { mn = fminf(mn, key[j]); mx = fmaxf(mx, key[j]); }
    wg_cnt_min_max(sh, cnt, mn, mx);
    if (cnt <= need) {  // the boundary bucket holds exactly the remainder: take it
      sel |= act;
      act = 0;
      break;
    }
    if (cnt <= kTopkThreads) {
      // exact ranking among the undecided candidates
      int mine = __popcll(act);
      int pos = mine ? atomicAdd(&sh.list_n, mine) : 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if ((act >> j) & 1ull) {
          sh.list_key[pos] = key[j];
          sh.list_idx[pos] = tid * PER + j;
          ++pos;
        }
      }
      __syncthreads();
      if (tid < cnt) {
        const float mk = sh.list_key[tid];
        const int mi = sh.list_idx[tid];
        int rank = 0;
        for (int u = 0; u < cnt; ++u) {
          const float ok = sh.list_key[u];
          const int oi = sh.list_idx[u];
          rank += (ok > mk) || (ok == mk && oi < mi);
        }
        if (rank < need) {
          const int b = geo.c0 + mi;
          atomicOr(&sh.bitmap[b >> 5], 1u << (b & 31));
        }
      }
      act = 0;
      break;
    }
    const float range = mx - mn;
    const float scale = 256.0f / range;
    if (!(range > 0.0f) || !(scale < __int_as_float(0x7f800000)) || it >= kTopkMaxIters) {
      robust = true;
      break;
    }
    sh.hist[tid] = 0;
    __syncthreads();
    int bk[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int b = (int)((key[j] - mn) * scale);
      b = b > 255 ? 255 : (b < 0 ? 0 : b);
      bk[j] = b;
      if ((act >> j) & 1ull) atomicAdd(&sh.hist[b], 1);
    }
    __syncthreads();
    if (tid < kWave) {
      // suffix counts over the 256 buckets, 4 per lane, in wave 0
      const int lane = tid;
      const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
      const int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
      int suf = h0 + h1 + h2 + h3;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_down(suf, o, kWave);
        if (lane + o < kWave) suf += n;
      }
      const int s3 = suf - h0 - h1 - h2;  // suffix count from bucket 4l+3
      const int s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
      int best = -1;
      if (s0 >= need) best = 4 * lane;
      if (s1 >= need) best = 4 * lane + 1;
      if (s2 >= need) best = 4 * lane + 2;
      if (s3 >= need) best = 4 * lane + 3;
      int bmax = best;
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) bmax = max(bmax, __shfl_xor(bmax, o, kWave));
      if (best == bmax && best >= 0) {
        const int sb = (best & 3) == 0 ? s0 : (best & 3) == 1 ? s1 : (best & 3) == 2 ? s2 : s3;
        sh.bstar = best;
        sh.cabove = sb - sh.hist[best];
      }
    }
    __syncthreads();
    const int bstar = sh.bstar, cabove = sh.cabove;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((act >> j) & 1ull) {
        if (bk[j] > bstar) { sel |= 1ull << j; act &= ~(1ull << j); }
        else if (bk[j] < bstar) { act &= ~(1ull << j); }
      }
    }
    need -= cabove;
    __syncthreads();
  }

  if (robust) {
    // threshold T = need-th largest integer key among the undecided, by bits
    uint32_t ukey[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) ukey[j] = score_key(key[j]);
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int c = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) c += ((act >> j) & 1ull) && ukey[j] >= cand;
      c = wg_sum(sh, c, 1);
      if (c >= need) prefix = cand;
    }
    uint64_t above = 0, equal = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((act >> j) & 1ull) {
        if (ukey[j] > prefix) above |= 1ull << j;
        else if (ukey[j] == prefix) equal |= 1ull << j;
      }
    }
    const int nabove = wg_sum(sh, __popcll(above), 1);
    sel |= above | lowest_index_fill<PER>(sh, equal, need - nabove);
  }

  // emit: forced blocks [0, c0) U [c1, nb) and the chosen candidates, ascending
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if ((sel >> j) & 1ull) {
      const int b = geo.c0 + tid * PER + j;
      atomicOr(&sh.bitmap[b >> 5], 1u << (b & 31));
    }
  }
  __syncthreads();
  constexpr int kWordsPerThread = (16384 / 32) / kTopkThreads;  // 2
  uint32_t words[kWordsPerThread];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kWordsPerThread; ++i) {
    const int w = tid * kWordsPerThread + i;
    uint32_t x = 0;
    if (w < nwords) {
      x = sh.bitmap[w];
      const int b0 = w * 32;
      // forced ranges, and nothing at or beyond nb
#pragma unroll 1
      for (int bb = 0; bb < 32; ++bb) {
        const int b = b0 + bb;
        if (b < geo.nb && (b < geo.c0 || b >= geo.c1)) x |= 1u << bb;
        if (b >= geo.nb) x &= ~(1u << bb);
      }
    }
    words[i] = x;
    mine += __popc(x);
  }
  int total;
  int pos = wg_excl_scan(sh, mine, 3, &total);
  int32_t* out = a.selected + ((size_t)r * a.num_kv_heads + g) * a.max_selected;
#pragma unroll
  for (int i = 0; i < kWordsPerThread; ++i) {
    uint32_t x = words[i];
    const int b0 = (tid * kWordsPerThread + i) * 32;
    while (x) {
      const int bb = __builtin_ctz(x);
      x &= x - 1;
      if (pos < a.max_selected) out[pos] = b0 + bb;
      ++pos;
    }
  }
  for (int i = total + tid; i < a.max_selected; i += kTopkThreads) out[i] = -1;
  if (tid == 0)
    a.selected_count[(size_t)r * a.num_kv_heads + g] = total < a.max_selected ? total : a.max_selected;
}

// One wave per (request, kv head), four per workgroup.
template <int MAXC>
__global__ __launch_bounds__(256) void topk_wave_kernel(TopkArgs a) {
  __shared__ WaveTopkLds<MAXC> sh[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.b.batch * a.num_kv_heads) return;
  const int r = item / a.num_kv_heads, g = item % a.num_kv_heads;
  const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
  const float* srow = a.scores + ((size_t)r * a.num_kv_heads + g) * a.b.max_blocks + geo.c0;
  topk_wave<MAXC>(srow, geo, topk_budget(a, geo), a.selected + (size_t)item * a.max_selected,
                  a.max_selected, a.selected_count + item, sh[wave], lane);
}

template <int MAXC>
static hipError_t launch_wave(const TopkArgs& a, hipStream_t st) {
  const int items = a.b.batch * a.num_kv_heads;
  hipLaunchKernelGGL((topk_wave_kernel<MAXC>), dim3((items + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int PER>
static hipError_t launch_wg(const TopkArgs& a, hipStream_t st) {
  dim3 grid(a.num_kv_heads, a.b.batch);
  hipLaunchKernelGGL((topk_wg_kernel<PER>), grid, dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int n = a.b.max_blocks;
  if (n <= 512) return launch_wave<512>(a, st);
  if (n <= 2048) return launch_wave<2048>(a, st);
  if (n <= 4096) return launch_wave<4096>(a, st);
  const int pwg = (n + kTopkThreads - 1) / kTopkThreads;
  if (pwg <= 32) return launch_wg<32>(a, st);
  return launch_wg<64>(a, st);
}

}  // namespace ls

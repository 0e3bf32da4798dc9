// The decode step planned from the lengths of the step (Vortex post, "Making
// it fast": the batch's sequence lengths are known when a step starts, so the
// work is planned and the workgroups balanced across requests of different
// lengths; ByteCross App. A: attention over disjoint token sets merged by
// log-sum-exp; §4.4: split-K).
//
// Three launches, no workgroup ever waits for another:
//   1. scoring: the pages that just filled get their summaries, then the
//      candidate summary tiles of all (request, kv head) pairs, laid out
//      flat in pair order, are cut into kPlanScoreGrid equal contiguous
//      ranges; each workgroup scores its range (which may span pairs) into
//      the pairs' score rows;
//   2. ranking: one workgroup per pair loads its row and takes the exact
//      top-k (the fast bucketed select over the known score range), plus the
//      forced blocks, into the selection;
//   3. attention: the selected positions of all pairs, laid out flat, are cut
//      into kPlanAttnGrid equal ranges; each workgroup attends its range 64
//      positions at a time, folding the passes' softmax states together in
//      registers. A pair inside one range is written out directly; a pair cut
//      by range ends leaves one state per workgroup in that workgroup's
//      slot, and the last of its workgroups to arrive merges them in range
//      order (device-coherent hand-off, arrival counter reset by that
//      workgroup, slots read back to zero).
// Every workgroup computes the plan itself: the per-pair counts (candidate
// tiles from the lengths, selection sizes from the counts) and their prefix
// sums, one pass for the total and one to find its range's pairs. The cut
// depends on nothing but those counts, so the results are deterministic and
// ls_sparse_decode_step equals ls_score_select + ls_sparse_attn_decode bit
// for bit.
#include "dev_item.h"
#include "dev_summary.h"
#include "dev_topk.h"
#include "ls_plan.h"

namespace ls {

namespace {

constexpr int NW = kPlanWaves;
constexpr int NT = kPlanThreads;
constexpr int kPlanMergeBatch = 4;   // slot states the merger loads per round
#ifndef LS_PLAN_PREFETCH
#define LS_PLAN_PREFETCH 2
#endif
#ifndef LS_PLAN_ATTN_WAVES_PER_EU
#define LS_PLAN_ATTN_WAVES_PER_EU 2
#endif
constexpr int kPlanPrefetch = LS_PLAN_PREFETCH;   // K/V blocks in flight per attention wave
#ifndef LS_PLAN_SCORE_PREFETCH
#define LS_PLAN_SCORE_PREFETCH 2
#endif
#ifndef LS_PLAN_SCORE_WAVES_PER_EU
#define LS_PLAN_SCORE_WAVES_PER_EU 4
#endif
constexpr int kPlanScorePrefetch = LS_PLAN_SCORE_PREFETCH;   // summary tiles in flight per wave
// What visiting one more pair costs a workgroup (its page ids or walk
// entries, its queries, the merge of its waves' states, its output), in
// items of the plan: 16-block summary tiles when scoring, positions (16-token
// blocks) when attending (measured on MI355X).
#ifndef LS_PLAN_SCORE_VISIT
#define LS_PLAN_SCORE_VISIT 4
#endif
#ifndef LS_PLAN_ATTN_VISIT
#define LS_PLAN_ATTN_VISIT 12
#endif
constexpr int kPlanScoreVisit = LS_PLAN_SCORE_VISIT;
constexpr int kPlanAttnVisit = LS_PLAN_ATTN_VISIT;

// Device-wide plan walk: the pairs' counts in pair order, this workgroup's
// range of the flat space, and the pairs that intersect it.
struct PlanWalkLds {
  int wtot[NW];         // per-wave totals of a scan
  int wcnt[NW];         // per-wave numbers of listed pairs
  int hit_p[NT];        // the chunk's pairs of the range, wave w's at [64 w, 64 w + wcnt[w])
  int hit_s[NT];
  int hit_n[NT];
};

// The flat space: pair p owns items [S_p, S_p + count(p) + C) (C more items
// when count(p) > 0: what visiting a pair costs beyond its own items, so
// that a range of many short pairs holds fewer items), S_p = the sum of the
// items of the pairs before it; T = the sum of all. Workgroup w of
// G = max(1, min(gridDim.x, T)) owns [w T / G, (w + 1) T / G) (every range
// is then non-empty unless T = 0; workgroups w >= G have none). For each
// pair whose items intersect the range, in pair order, the whole workgroup
// calls visit(p, S_p, count(p), lo, hi, T, G) (the pair's items: count(p) +
// C from S_p); with kEmpty, also for each empty pair whose S_p the range
// holds (S_p = T: the last range).
// count(p) is called by one thread per pass; it must return the same value
// each time, with T < 2^31. Pass 1 sums the counts over the workgroup;
// pass 2 scans them NT pairs at a time (one count per thread, a workgroup
// prefix sum) and lists the pairs of the range.
template <bool kEmpty, int C, class Count, class Visit>
__device__ void plan_walk(int pairs, PlanWalkLds& sh, Count count, Visit visit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  // pass 1: the total
  auto items = [&](int n) { return n > 0 ? n + C : 0; };
  int mine = 0;
  for (int p = tid; p < pairs; p += NT) mine += items(count(p));
  {
    const int incl = wave_incl_scan_dpp(mine);
    if (lane == 63) sh.wtot[wave] = incl;
  }
  __syncthreads();
  int T = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) T += sh.wtot[w];
  T = __builtin_amdgcn_readfirstlane(T);   // uniform: keep it (and what follows) scalar
  __syncthreads();   // wtot is rewritten by pass 2
  const int G = T < 1 ? 1 : ((int)gridDim.x < T ? (int)gridDim.x : T);
  const int w = blockIdx.x;
  if (w >= G) return;
  const int lo = (int)((long long)w * T / G), hi = (int)((long long)(w + 1) * T / G);
  // pass 2: the pairs of [lo, hi), NT at a time
  int base = 0;   // S of the chunk's first pair
  for (int c = 0; c < pairs; c += NT) {
    const int p = c + tid;
    const int n = p < pairs ? count(p) : 0;
    const int ni = items(n);
    const int incl = wave_incl_scan_dpp(ni);
    if (lane == 63) sh.wtot[wave] = incl;
    __syncthreads();
    int pre = 0, ctot = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int v = sh.wtot[u];
      pre += u < wave ? v : 0;
      ctot += v;
    }
    const int s = base + pre + incl - ni;
    const bool hit = n > 0 ? (s < hi && s + ni > lo)
                           : (kEmpty && p < pairs && ((s >= lo && s < hi) || (s == T && w == G - 1)));
    const unsigned long long m = __ballot(hit);
    if (hit) {
      const int i = wave * kWave + mbcnt(m);
      sh.hit_p[i] = p;
      sh.hit_s[i] = s;
      sh.hit_n[i] = n;
    }
    if (lane == 0) sh.wcnt[wave] = __popcll(m);
    __syncthreads();
    for (int u = 0; u < NW; ++u) {
      const int nh = __builtin_amdgcn_readfirstlane(sh.wcnt[u]);
      for (int i = 0; i < nh; ++i) {
        const int j = u * kWave + i;
        visit(__builtin_amdgcn_readfirstlane(sh.hit_p[j]), __builtin_amdgcn_readfirstlane(sh.hit_s[j]),
              __builtin_amdgcn_readfirstlane(sh.hit_n[j]), lo, hi, T, G);
      }
    }
    __syncthreads();   // the lists and wtot are rewritten by the next chunk
    base += __builtin_amdgcn_readfirstlane(ctot);
    // later pairs start at or past hi: none is ours, except empty pairs at T
    // for the last range
    if (base >= hi && !(kEmpty && hi == T)) break;
  }
}

// ------------------------------------------------------------- scoring ----

template <int D>
struct ScoreLds {
  PlanWalkLds walk;
  int pg[kPlanSubTiles * 16];
  alignas(16) uint32_t stage[NW * 2 * 16 * Stage<D>::kKRowWords];
};

// Candidate tiles of a request: tiles [c0 / 16, ceil(c1 / 16)).
__device__ __forceinline__ int cand_tiles(const ReqGeom& geo) {
  return geo.c1 > geo.c0 ? (geo.c1 + 15) / 16 - geo.c0 / 16 : 0;
}

template <int D, bool kBounds>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(LS_PLAN_SCORE_WAVES_PER_EU)))
void plan_score_kernel(PlanArgs f) {
  __shared__ ScoreLds<D> sh;
  const ScoreArgs& sa = f.sa;
  const int tid = threadIdx.x, HKV = sa.num_kv_heads;
  // the pages that just filled: one wave per (page, kv head) tile (they are
  // recent blocks, never scored in this call)
  for (int tile = blockIdx.x * NW + wave_id(); tile < f.up.n_tiles; tile += gridDim.x * NW) {
    if constexpr (kBounds)
      bounds_tile_bf16<D>(f.up.keys, f.up.pages, tile, sa.b.num_pages, HKV, sa.b.page_size,
                          static_cast<uint16_t*>(f.up.out));
    else
      summary_tile_bf16<D, false>(f.up.keys, f.up.pages, tile, sa.b.num_pages, HKV,
                                  sa.b.page_size, f.up.out);
  }
  auto count = [&](int p) {
    return cand_tiles(req_geom(sa.b, p / HKV, sa.n_sink, sa.n_recent));
  };
  auto visit = [&](int p, int s, int n, int lo, int hi, int, int) {
    const int r = p / HKV, g = p - r * HKV;
    const ReqGeom geo = req_geom(sa.b, r, sa.n_sink, sa.n_recent);
    const int t0 = geo.c0 / 16;
    const int ta = (lo > s ? lo : s) - s, te = (hi < s + n ? hi : s + n) - s;   // ta >= te:
    float* row = f.rows + (size_t)p * sa.b.max_blocks;                          // none
    for (int a = ta; a < te; a += kPlanSubTiles) {
      const int b = te < a + kPlanSubTiles ? te : a + kPlanSubTiles;
      ReqGeom cg = geo;
      cg.c0 = geo.c0 > 16 * (t0 + a) ? geo.c0 : 16 * (t0 + a);
      cg.c1 = geo.c1 < 16 * (t0 + b) ? geo.c1 : 16 * (t0 + b);
      for (int i = tid; i < cg.c1 - cg.c0; i += NT) sh.pg[i] = sa.b.indices[geo.page_base + cg.c0 + i];
      __syncthreads();
      if constexpr (kBounds)
        item_score_bounds<D, kPlanMaxBlocks, kStoreGlobal, NW>(sa, r, g, cg, sh.pg, row, sh.stage,
                                                               nullptr, cg.c0);
      else
        item_score<D, kPlanMaxBlocks, kStoreGlobal, NW, kPlanScorePrefetch>(
            sa, r, g, cg, sh.pg, row, sh.stage, nullptr, cg.c0);
      __syncthreads();   // pg and the staging tiles are reused
    }
  };
  plan_walk<false, kPlanScoreVisit>(f.pairs, sh.walk, count, visit);
}

// ------------------------------------------------------------- ranking ----

template <int MAXC>
struct RankLds {
  alignas(16) float sc[MAXC + MAXC / 16];   // the candidates' scores, padded row
  TopkFastLds<MAXC> tf;
  TopkLds tk;
  float red[2][kPlanRankThreads / kWave];
};

template <int MAXC>
__global__ __launch_bounds__(kPlanRankThreads)
__attribute__((amdgpu_waves_per_eu(MAXC <= 8192 ? 4 : 2))) void plan_rank_kernel(PlanArgs f) {
  constexpr int RT = kPlanRankThreads, RW = RT / kWave, NPT = MAXC / RT;
  __shared__ RankLds<MAXC> sh;
  const TopkArgs& ta = f.ta;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int pair = blockIdx.x;
  const int r = pair / ta.num_kv_heads;
  const ReqGeom geo = req_geom(ta.b, r, ta.n_sink, ta.n_recent);
  const int nc = geo.c1 - geo.c0;
  float* row = f.rows + (size_t)pair * ta.b.max_blocks + geo.c0;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  constexpr int CH = NPT < 8 ? NPT : 8;   // loads in flight per thread
#pragma unroll
  for (int m0 = 0; m0 < NPT; m0 += CH) {
    float v[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int e = tid + (m0 + u) * RT;
      v[u] = e < nc ? row[e] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int e = tid + (m0 + u) * RT;
      if (e < nc) {
        sh.sc[e + (e >> 4)] = v[u];
        mn = fminf(mn, v[u]);
        mx = fmaxf(mx, v[u]);
        if (f.zero_rows) row[e] = 0.0f;
      }
    }
  }
  mn = wave_min_fast(mn);
  mx = wave_max_fast(mx);
  if (lane == 0) {
    sh.red[0][wave] = mn;
    sh.red[1][wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    mn = fminf(mn, sh.red[0][w]);
    mx = fmaxf(mx, sh.red[1][w]);
  }
  int32_t* sel = ta.selected + (size_t)pair * ta.max_selected;
  int32_t* ent = f.ents ? f.ents + (size_t)pair * ta.max_selected : nullptr;
  const int32_t* pages = ta.b.indices + geo.page_base;
  auto emit = [&](int p, int b) {
    sel[p] = b;
    if (ent && b >= 0) {   // the attention's walk entry of position p (never 0); the
                           // positions past the selection are never read, left 0
      int e = -1;
      if (b >= 0 && b < geo.nb) {
        const int pg = pages[b];
        const int nt = geo.L - b * 16 < 16 ? geo.L - b * 16 : 16;
        if (pg >= 0 && pg < ta.b.num_pages && nt > 0) e = pg * 32 + nt;
      }
      ent[p] = e;
    }
  };
  const int stored = topk_fast<NPT, RT>(sh.sc, geo, topk_budget(ta, geo), ta.max_selected, sh.tf,
                                        sh.tk, sel, ta.selected_count + pair, mn, mx, emit);
  if (tid == 0) ta.selected_count[pair] = stored;
}

// ----------------------------------------------------------- attention ----

template <int D>
struct AttnLds {
  PlanWalkLds walk;
  int ent[kPlanSubPositions + item_entry_pad<NW>()];
  int flag;
  ItemAttnLds<D, NW> at;
};

// Folds state (m, o, l) into (M, O, L) (online log-sum-exp, log2 domain).
__device__ __forceinline__ void fold_state(float& M, float& O, float& L, float m, float o,
                                           float l) {
  const float Mn = fmaxf(M, m);
  if (Mn == kNegInf) return;
  const float fa = exp2_fast(M - Mn), fb = exp2_fast(m - Mn);   // -inf -> 0
  O = O * fa + o * fb;
  L = L * fa + l * fb;
  M = Mn;
}

// Counts one arrival at *ctr (device scope); true for the n-th, which also
// resets the counter. Called by one thread after the hand-off stores have
// completed.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, int n) {
  const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool last = prev == (uint32_t)(n - 1);
  if (last) st_dev(ctr, 0u);
  return last;
}

// The workgroup of the flat space [0, T) cut into G ranges that holds item x.
__device__ __forceinline__ int range_of(int x, int T, int G) {
  return (int)(((long long)(x + 1) * G - 1) / T);
}
__device__ __forceinline__ int range_lo(int w, int T, int G) {
  return (int)((long long)w * T / G);
}

template <int D, bool kDense>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(LS_PLAN_ATTN_WAVES_PER_EU)))
void plan_attn_kernel(PlanArgs f) {
  __shared__ AttnLds<D> sh;
  constexpr int EPT = item_ept<D, NW>();
  const AttnArgs& a = f.aa;
  const int tid = threadIdx.x, HKV = a.num_kv_heads;
  const bool out32 = a.out_dtype == LS_DTYPE_FP32;
  auto count = [&](int p) {
    if constexpr (kDense) {
      return req_geom(a.b, p / HKV, 0, 0).nb;
    } else {
      const int c = a.selected_count[p];
      return c < 0 ? 0 : (c > a.max_selected ? a.max_selected : c);
    }
  };
  // the output of the pair's 4 heads from a state of the element layout
  auto write_out = [&](int r, int g, const float* M, const float* O, const float* L) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + j * NT;
      if (e < 4 * D) {
        const int h = e / D, d = e - h * D;
        const float inv = L[j] > 0.0f ? 1.0f / L[j] : 0.0f;
        const size_t idx = ((size_t)r * a.num_q_heads + g * 4 + h) * D + d;
        if (out32) reinterpret_cast<float*>(a.out)[idx] = O[j] * inv;
        else reinterpret_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_rne(O[j] * inv);
        if (a.lse && d == 0)
          a.lse[(size_t)r * a.num_q_heads + g * 4 + h] =
              (M[j] == kNegInf || !(L[j] > 0.0f)) ? kNegInf : (M[j] + log2f(L[j])) * kLn2;
      }
    }
  };
  auto visit = [&](int p, int s, int n, int lo, int hi, int T, int G) {
    const int r = p / HKV, g = p - r * HKV;
    const ReqGeom geo = req_geom(a.b, r, 0, 0);
    const int32_t* pages = a.b.indices + geo.page_base;
    const int32_t* srow = kDense ? nullptr : a.selected + (size_t)p * a.max_selected;
    int32_t* erow = kDense || !f.ents ? nullptr : f.ents + (size_t)p * a.max_selected;
    const int pa = (lo > s ? lo : s) - s, pe = (hi < s + n ? hi : s + n) - s;
    float M[EPT], O[EPT], L[EPT];   // the running state of the pair's passes
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      M[j] = kNegInf;
      O[j] = 0.0f;
      L[j] = 0.0f;
    }
    for (int q0 = pa; q0 < pe; q0 += kPlanSubPositions) {
      const int cnt = pe - q0 < kPlanSubPositions ? pe - q0 : kPlanSubPositions;
      for (int pos = tid; pos < item_entry_count<NW>(cnt); pos += NT) {
        int e = -1;
        if (pos < cnt) {
          if (!kDense && erow) {   // written by the ranker (one load), reset to 0
            e = erow[q0 + pos];
            erow[q0 + pos] = 0;
          } else {
            const int blk = kDense ? q0 + pos : srow[q0 + pos];
            if (blk >= 0 && blk < geo.nb) {
              const int pg = pages[blk];
              const int nt = geo.L - blk * 16 < 16 ? geo.L - blk * 16 : 16;
              if (pg >= 0 && pg < a.b.num_pages && nt > 0) e = pg * 32 + nt;
            }
          }
        }
        sh.ent[pos] = e;
      }
      __syncthreads();
      ItemState<EPT> st;
      item_attn<D, false, NW, kSplitPlain, kPlanPrefetch>(a, r, g, sh.ent, cnt, sh.at, nullptr,
                                                          nullptr, &st);
#pragma unroll
      for (int j = 0; j < EPT; ++j) fold_state(M[j], O[j], L[j], st.m[j], st.o[j], st.l[j]);
      __syncthreads();   // the entries and the attention LDS are reused
    }
    const int ni = n > 0 ? n + kPlanAttnVisit : 0;   // the pair's items in the plan
    if (lo <= s && s + ni <= hi) {   // the whole pair is in this range (or it is empty)
      write_out(r, g, M, O, L);
      return;
    }
    // a part: publish it in this workgroup's slot, count the arrival
    const int w = blockIdx.x;
    const size_t sw = (size_t)4 * (D + 2);
    float* mine = f.slots + (lo >= s ? 2 * w : 2 * w + 1) * sw;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + j * NT;
      if (e < 4 * D) {
        const int h = e / D, d = e - h * D;
        st_dev(mine + h * (D + 2) + d, O[j]);
        if (d == 0) {
          st_dev(mine + h * (D + 2) + D, M[j]);
          st_dev(mine + h * (D + 2) + D + 1, L[j]);
        }
      }
    }
    wait_stores();   // this thread's words have reached the device-coherent level
    __syncthreads();
    const int w0 = range_of(s, T, G), w1 = range_of(s + ni - 1, T, G);
    if (tid == 0) sh.flag = arrive_last(f.ctl + kPlanCtlWords + p, w1 - w0 + 1);
    __syncthreads();
    if (!sh.flag) return;
    // the last to arrive: merge the parts in range order, reading each back to zero
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      M[j] = kNegInf;
      O[j] = 0.0f;
      L[j] = 0.0f;
    }
    for (int v0 = w0; v0 <= w1; v0 += kPlanMergeBatch) {
      float wo[kPlanMergeBatch][EPT], wm[kPlanMergeBatch][EPT], wl[kPlanMergeBatch][EPT];
#pragma unroll
      for (int u = 0; u < kPlanMergeBatch; ++u) {   // every load issued before the uses
        const int v = v0 + u;
        const float* ps = f.slots + (range_lo(v, T, G) >= s ? 2 * v : 2 * v + 1) * sw;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          const int e = tid + j * NT;
          wo[u][j] = 0.0f;
          wm[u][j] = kNegInf;
          wl[u][j] = 0.0f;
          if (v <= w1 && e < 4 * D) {
            const int h = e / D, d = e - h * D;
            wo[u][j] = ld_dev(ps + h * (D + 2) + d);
            wm[u][j] = ld_dev(ps + h * (D + 2) + D);
            wl[u][j] = ld_dev(ps + h * (D + 2) + D + 1);
          }
        }
      }
      __syncthreads();   // every thread of a head has read its (m, l) words
#pragma unroll
      for (int u = 0; u < kPlanMergeBatch; ++u) {
        const int v = v0 + u;
        float* ps = f.slots + (range_lo(v, T, G) >= s ? 2 * v : 2 * v + 1) * sw;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          const int e = tid + j * NT;
          if (v <= w1 && e < 4 * D) {
            const int h = e / D, d = e - h * D;
            st_dev(ps + h * (D + 2) + d, 0.0f);
            if (d == 0) {
              st_dev(ps + h * (D + 2) + D, 0.0f);
              st_dev(ps + h * (D + 2) + D + 1, 0.0f);
            }
            fold_state(M[j], O[j], L[j], wm[u][j], wo[u][j], wl[u][j]);
          }
        }
      }
    }
    write_out(r, g, M, O, L);
  };
  plan_walk<true, kPlanAttnVisit>(f.pairs, sh.walk, count, visit);
}

hipError_t launch_rank(const PlanArgs& p, hipStream_t st) {
  const int n = p.max_blocks;
  const dim3 grid(p.pairs), block(kPlanRankThreads);
  if (n <= 2048) hipLaunchKernelGGL((plan_rank_kernel<2048>), grid, block, 0, st, p);
  else if (n <= 4096) hipLaunchKernelGGL((plan_rank_kernel<4096>), grid, block, 0, st, p);
  else if (n <= 8192) hipLaunchKernelGGL((plan_rank_kernel<8192>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((plan_rank_kernel<16384>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan_select(const PlanArgs& p, hipStream_t st) {
  if (p.pairs <= 0) return hipSuccess;
  const dim3 grid(kPlanScoreGrid), block(NT);
  const bool b = p.sa.bounds != 0;
  if (p.sa.head_dim == 128) {
    if (b) hipLaunchKernelGGL((plan_score_kernel<128, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((plan_score_kernel<128, false>), grid, block, 0, st, p);
  } else {
    if (b) hipLaunchKernelGGL((plan_score_kernel<64, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((plan_score_kernel<64, false>), grid, block, 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rank(p, st);
}

hipError_t launch_plan_attend(const PlanArgs& p, hipStream_t st) {
  if (p.pairs <= 0) return hipSuccess;
  const dim3 grid(kPlanAttnGrid), block(NT);
  const bool dense = p.aa.selected == nullptr;
  if (p.aa.head_dim == 128) {
    if (dense) hipLaunchKernelGGL((plan_attn_kernel<128, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((plan_attn_kernel<128, false>), grid, block, 0, st, p);
  } else {
    if (dense) hipLaunchKernelGGL((plan_attn_kernel<64, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((plan_attn_kernel<64, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace ls

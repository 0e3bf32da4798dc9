// The decode step spread over the whole chip (Vortex post, "Making it fast":
// the operators of one step fused; ByteCross App. A: attention over disjoint
// token sets merged by log-sum-exp; §4.4: split-K).
//
// One launch, one 256-thread workgroup per work item, items in blockIdx order:
//   1. refresh items: the summaries (or Quest bounds) of pages that just
//      filled, one wave per (page, kv head) tile;
//   2. score items: chunk c of the candidate tiles of pair (request r, kv
//      head g) -- the block scores go to the pair's score row in HBM and the
//      chunk's score range next to it; the LAST chunk of the pair to finish
//      (a per-pair arrival counter) ranks the whole row (top-k + forced
//      blocks), writes the selection and raises the pair's ready flag;
//   3. attention items: split s of the pair's selection positions -- wait
//      for the ready flag, attend, write the split's softmax state (m, l, o);
//      the LAST split of the pair to finish merges the pair's splits in split
//      order and writes the output.
// Every hand-off inside the launch (scores, ranges, selection, split states)
// uses device-coherent stores and loads; the per-XCD L2s are never flushed.
// Nothing depends on the order in which workgroups finish, so the results are
// deterministic. An attention item waits only for score items of lower index:
// the dispatcher starts workgroups in index order on each XCD, so a waited-on
// item has started before its waiter and makes progress while it waits. The
// wait is still bounded: past kFlowSpinLimit polls it gives up and raises the
// error word (results then unspecified).
//
// Control words (per pair: score arrivals, split arrivals, ready flag; one
// error word) start at zero and every call leaves them at zero: the last
// arriver of each counter resets it, the last split resets the ready flag.
//
// The select-only form (no attention items) serves ls_score_select, the
// attention-only form (no score items, no waiting) ls_sparse_attn_decode, so
// that the step and the separate calls give the same bits.
#include "dev_item.h"
#include "dev_summary.h"
#include "ls_flow.h"

namespace ls {

namespace {

constexpr int NW = kFlowWaves;
constexpr int NT = kFlowThreads;

template <int D, int MAXC>
struct FlowLds {
  int pg[kFlowMaxChunkBlocks];                      // score item: the chunk's page ids
  int ent[kFlowMaxSplit + item_entry_pad<NW>()];    // attention item: walk entries
  float rng[2 * kFlowMaxChunks];                    // top-k: chunk score ranges
  int flag;
  union {
    struct {
      alignas(16) uint32_t stage[NW * 2 * 16 * Stage<D>::kKRowWords];
      float range[2 * NW];
    } s;
    struct {
      alignas(16) float sc[MAXC + MAXC / 16];       // padded score row
      TopkLds tk;
      TopkFastLds tf;
      int pgrow[kFlowEntries<MAXC> ? MAXC : 1];     // the pair's page-table row
      int sel[kFlowEntries<MAXC> ? MAXC : 1];       // the selection
    } t;
    ItemAttnLds<D, NW> at;
  } u;
};

__device__ __forceinline__ uint32_t atomic_inc_dev(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Chunk c of pair `pair`: score its candidates, publish its range, count the
// arrival; the last arrival ranks the pair.
template <int D, int MAXC, bool kBounds, bool kAttn>
__device__ void flow_score(const FlowArgs& f, int item, FlowLds<D, MAXC>& sh) {
  const ScoreArgs& sa = f.sa;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int pair = item / f.chunks, c = item - pair * f.chunks;
  const int r = pair / sa.num_kv_heads, g = pair - r * sa.num_kv_heads;
  const ReqGeom geo = req_geom(sa.b, r, sa.n_sink, sa.n_recent);
  // the chunk: tiles [tb, tb + tiles_per_chunk) of the candidate range
  const int tb = geo.c0 / 16 + c * f.chunk_tiles;
  ReqGeom cg = geo;
  cg.c0 = geo.c0 > 16 * tb ? geo.c0 : 16 * tb;
  cg.c1 = geo.c1 < 16 * (tb + f.chunk_tiles) ? geo.c1 : 16 * (tb + f.chunk_tiles);
  if (cg.c1 < cg.c0) cg.c1 = cg.c0;
  const int n = cg.c1 - cg.c0;   // <= kFlowMaxChunkBlocks
  for (int i = tid; i < n; i += NT) sh.pg[i] = sa.b.indices[geo.page_base + cg.c0 + i];
  __syncthreads();
  float* row = f.score_rows + (size_t)pair * sa.b.max_blocks;
  if (n > 0) {
    if constexpr (kBounds)
      item_score_bounds<D, MAXC, kStoreDev, NW>(sa, r, g, cg, sh.pg, row, sh.u.s.stage,
                                                sh.u.s.range, cg.c0);
    else
      item_score<D, MAXC, kStoreDev, NW>(sa, r, g, cg, sh.pg, row, sh.u.s.stage, sh.u.s.range,
                                         cg.c0);
  } else if (lane == 0) {
    sh.u.s.range[wave] = __builtin_huge_valf();
    sh.u.s.range[NW + wave] = -__builtin_huge_valf();
  }
  __syncthreads();
  if (tid == 0) {
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mn = fminf(mn, sh.u.s.range[w]);
      mx = fmaxf(mx, sh.u.s.range[NW + w]);
    }
    float* rg = f.ranges + ((size_t)pair * kFlowMaxChunks + c) * 2;
    st_dev(rg, mn);
    st_dev(rg + 1, mx);
  }
  wait_stores();   // this thread's scores and range have reached the coherent level
  __syncthreads();
  uint32_t* ctl = f.ctl + (size_t)pair * kFlowCtlPerPair;
  if (tid == 0) {
    const bool last = atomic_inc_dev(&ctl[kCtlScoreArrivals]) == (uint32_t)(f.chunks - 1);
    if (last) st_dev(&ctl[kCtlScoreArrivals], 0u);
    sh.flag = last;
  }
  __syncthreads();
  if (!sh.flag) return;

  // ---- the pair's top-k: the whole score row, every chunk's range ----
  // (raised wave priority: the ranking is on the pair's critical path, the
  // streaming workgroups sharing the CU are not)
  __builtin_amdgcn_s_setprio(3);
  constexpr bool kEnt = kAttn && kFlowEntries<MAXC>;
  const int nc = geo.c1 - geo.c0;
  constexpr int NPT = MAXC / NT;
  float v[NPT];
  int pv[kEnt ? NPT : 1];
#pragma unroll
  for (int m = 0; m < NPT; ++m) {   // every load issued before the stores
    const int e = tid + m * NT;
    v[m] = e < nc ? ld_dev(&row[geo.c0 + e]) : 0.0f;
    // with the scores, the pair's page-table row (for the walk entries)
    if constexpr (kEnt) pv[m] = e < geo.nb ? sa.b.indices[geo.page_base + e] : 0;
  }
  for (int w = tid; w < f.chunks; w += NT) {
    const float* rg = f.ranges + ((size_t)pair * kFlowMaxChunks + w) * 2;
    sh.rng[w] = ld_dev(rg);
    sh.rng[f.chunks + w] = ld_dev(rg + 1);
  }
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int e = tid + m * NT;
    if (e < nc) sh.u.t.sc[e + (e >> 4)] = v[m];
    if constexpr (kEnt) {
      if (e < geo.nb) sh.u.t.pgrow[e] = pv[m];
    }
  }
  __syncthreads();
  const TopkArgs& ta = f.ta;
  int cnt;
  if constexpr (MAXC <= kTopkFastMaxBlocks) {
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    for (int w = 0; w < f.chunks; ++w) {
      mn = fminf(mn, sh.rng[w]);
      mx = fmaxf(mx, sh.rng[f.chunks + w]);
    }
    cnt = topk_fast<NPT, NT, kAttn>(sh.u.t.sc, geo, topk_budget(ta, geo),
                                    ta.selected + (size_t)pair * ta.max_selected,
                                    ta.max_selected, ta.selected_count + pair, sh.u.t.tf,
                                    sh.u.t.tk, kEnt ? sh.u.t.sel : nullptr, mn, mx);
  } else {
    cnt = topk_wg<NPT, NT, true, kAttn>(sh.u.t.sc, geo, topk_budget(ta, geo),
                                        ta.selected + (size_t)pair * ta.max_selected,
                                        ta.max_selected, ta.selected_count + pair, sh.u.t.tk,
                                        kEnt ? sh.u.t.sel : nullptr, sh.rng, f.chunks);
  }
  if constexpr (kEnt) {
    // walk entries of the selection (page * 32 + valid tokens), so that the
    // attention items need no page-table lookup of their own
    int32_t* ent = f.ents + (size_t)pair * ta.max_selected;
    for (int i = tid; i < cnt; i += NT) {
      const int blk = sh.u.t.sel[i];
      int e = -1;
      if (blk >= 0 && blk < geo.nb) {
        const int p = sh.u.t.pgrow[blk];
        const int nt = geo.L - blk * 16 < 16 ? geo.L - blk * 16 : 16;
        if (p >= 0 && p < sa.b.num_pages && nt > 0) e = p * 32 + nt;
      }
      st_dev(&ent[i], e);
    }
  }
  if constexpr (kAttn) {
    wait_stores();   // the selection, its count and entries are visible device-wide
    __syncthreads();
    if (tid == 0) st_dev(&ctl[kCtlReady], 1u);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Split s of pair `pair`: wait for its selection (kScore), attend positions
// [s * split, s * split + split) of it, publish the state, count the
// arrival; the last arrival merges the pair's splits.
template <int D, int MAXC, bool kScore>
__device__ void flow_attn(const FlowArgs& f, int item, FlowLds<D, MAXC>& sh) {
  const AttnArgs& a = f.aa;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int pair = item / f.splits, s = item - pair * f.splits;
  const int r = pair / a.num_kv_heads, g = pair - r * a.num_kv_heads;
  uint32_t* ctl = f.ctl + (size_t)pair * kFlowCtlPerPair;
  if constexpr (kScore) {
    if (tid == 0) {
      int spins = 0;
      while (ld_dev(&ctl[kCtlReady]) == 0u) {
        if (++spins > kFlowSpinLimit) {
          st_dev(f.ctl + (size_t)f.pairs * kFlowCtlPerPair + kCtlError, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
  }
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  int total = ld_x<kScore>(&a.selected_count[pair]);
  total = total < 0 ? 0 : (total > a.max_selected ? a.max_selected : total);
  const int p0 = s * f.split;
  int cnt = total - p0;
  cnt = cnt < 0 ? 0 : (cnt > f.split ? f.split : cnt);
  const int32_t* srow = a.selected + (size_t)pair * a.max_selected + p0;
  const int32_t* pages = a.b.indices + geo.page_base;
  constexpr bool kEnt = kScore && kFlowEntries<MAXC>;
  const int32_t* erow = kEnt ? f.ents + (size_t)pair * a.max_selected + p0 : nullptr;
  for (int pos = tid; pos < item_entry_count<NW>(cnt); pos += NT) {
    int e = -1;
    if (pos < cnt) {
      if constexpr (kEnt) {
        e = ld_dev(&erow[pos]);   // written by the pair's ranking workgroup
      } else {
        const int blk = ld_x<kScore>(&srow[pos]);
        if (blk >= 0 && blk < geo.nb) {
          const int p = pages[blk];
          const int nt = geo.L - blk * 16 < 16 ? geo.L - blk * 16 : 16;
          if (p >= 0 && p < a.b.num_pages && nt > 0) e = p * 32 + nt;
        }
      }
    }
    sh.ent[pos] = e;
  }
  __syncthreads();
  const ItemSplit sp{f.parts, f.splits, s};
  if (cnt > 0) {
    item_attn<D, false, NW, true, 1>(a, r, g, sh.ent, cnt, sh.u.at, nullptr, &sp);
  } else {
    // an empty split: m = -inf, l = 0, o = 0
    for (int e = tid; e < 4 * (D + 2); e += NT) {
      const int h = e / (D + 2), d = e - h * (D + 2);
      float* ph = f.parts + (((size_t)r * a.num_q_heads + g * 4 + h) * f.splits + s) * (D + 2);
      st_dev(ph + d, d == D ? kNegInf : 0.0f);
    }
  }
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const bool last = atomic_inc_dev(&ctl[kCtlSplitArrivals]) == (uint32_t)(f.splits - 1);
    if (last) {
      st_dev(&ctl[kCtlSplitArrivals], 0u);
      if (kScore) st_dev(&ctl[kCtlReady], 0u);   // every split of the pair has waited
    }
    sh.flag = last;
  }
  __syncthreads();
  if (!sh.flag) return;
  // one wave per query head of the group, splits merged in split order
  __builtin_amdgcn_s_setprio(3);
  AttnArgs m = a;
  m.partials = f.parts;
  m.num_splits = f.splits;
  combine_head<D, true>(m, r * a.num_q_heads + g * 4 + wave, lane);
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int MAXC, bool kBounds, bool kScore, bool kAttn>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(MAXC <= 4096 ? 4 : 2))) void flow_kernel(FlowArgs f) {
  __shared__ FlowLds<D, MAXC> sh;
  int item = blockIdx.x;
  if (item < f.n_refresh) {
    const int tile = item * NW + wave_id();
    if (tile < f.up.n_tiles) {
      if constexpr (kBounds)
        bounds_tile_bf16<D>(f.up.keys, f.up.pages, tile, f.sa.b.num_pages, f.sa.num_kv_heads,
                            f.sa.b.page_size, static_cast<uint16_t*>(f.up.out));
      else
        summary_tile_bf16<D, false>(f.up.keys, f.up.pages, tile, f.sa.b.num_pages,
                                    f.sa.num_kv_heads, f.sa.b.page_size, f.up.out);
    }
    return;
  }
  item -= f.n_refresh;
  if constexpr (kScore) {
    if (item < f.pairs * f.chunks) {
      flow_score<D, MAXC, kBounds, kAttn>(f, item, sh);
      return;
    }
    item -= f.pairs * f.chunks;
  }
  if constexpr (kAttn) {
    if (item < f.pairs * f.splits) flow_attn<D, MAXC, kScore>(f, item, sh);
  }
}

template <int D, int MAXC, bool kBounds, bool kScore, bool kAttn>
hipError_t launch_flow_t(const FlowArgs& f, hipStream_t st) {
  const int items = f.n_refresh + (kScore ? f.pairs * f.chunks : 0) +
                    (kAttn ? f.pairs * f.splits : 0);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL((flow_kernel<D, MAXC, kBounds, kScore, kAttn>), dim3(items), dim3(NT), 0,
                     st, f);
  return hipGetLastError();
}

template <int D, int MAXC>
hipError_t launch_flow_d(const FlowArgs& f, int mode, hipStream_t st) {
  const bool bounds = f.sa.bounds != 0;
  switch (mode) {
    case kFlowSelect:
      return bounds ? launch_flow_t<D, MAXC, true, true, false>(f, st)
                    : launch_flow_t<D, MAXC, false, true, false>(f, st);
    case kFlowAttend:
      return launch_flow_t<D, MAXC, false, false, true>(f, st);
    default:
      return bounds ? launch_flow_t<D, MAXC, true, true, true>(f, st)
                    : launch_flow_t<D, MAXC, false, true, true>(f, st);
  }
}

}  // namespace

hipError_t launch_flow(const FlowArgs& f, int mode, hipStream_t st) {
  const int D = f.sa.head_dim > 0 ? f.sa.head_dim : f.aa.head_dim;
  const int n = f.max_blocks;
  if (D == 128) {
    if (n <= 2048) return launch_flow_d<128, 2048>(f, mode, st);
    if (n <= 4096) return launch_flow_d<128, 4096>(f, mode, st);
    return launch_flow_d<128, 8192>(f, mode, st);
  }
  if (n <= 2048) return launch_flow_d<64, 2048>(f, mode, st);
  if (n <= 4096) return launch_flow_d<64, 4096>(f, mode, st);
  return launch_flow_d<64, 8192>(f, mode, st);
}

}  // namespace ls

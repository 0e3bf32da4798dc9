// The decode step spread over the whole chip (Vortex post, "Making it fast":
// the operators of one step fused; ByteCross App. A: attention over disjoint
// token sets merged by log-sum-exp; §4.4: split-K).
//
// One launch, one 256-thread workgroup per work item, items in blockIdx order:
//   1. refresh items: the summaries (or Quest bounds) of pages that just
//      filled, one wave per (page, kv head) tile;
//   2. score items: chunk c of the candidate tiles of pair (request r, kv
//      head g); the block scores go to the pair's key row in HBM as
//      order-preserving keys, and the chunk counts its arrival. The LAST chunk
//      of the pair to arrive (the ranker) loads the row, ranks the pair
//      (top-k + forced blocks), writes the selection and publishes the
//      selection's walk entries (page * 32 + valid tokens, never 0);
//   3. attention items: split s of the pair's selection positions -- poll
//      the split's walk entries until they are written, attend, publish the
//      split's softmax state (m, l, o) and count the arrival; the LAST split
//      of the pair to arrive merges the states in split order into the
//      output.
// Stores handed to another workgroup are device-coherent and complete
// before the arrival is counted (no cache-wide fences). Every word a call
// hands over is reset to zero by its reader (arrival counters by the last
// arrival), so the workspace is zero again after the call. An attention item
// waits only for score items of lower index, which the dispatcher starts
// first on each XCD; the wait still gives up after kFlowSpinLimit polls and
// raises the error word (results then unspecified). Nothing depends on the
// order in which workgroups finish, so the results are deterministic.
//
// The select-only form (no attention items) serves ls_score_select, the
// attention-only form (walk entries from the given selection, no waiting
// for them) ls_sparse_attn_decode; both use the same chunking, kernel code
// and merge order as the step, so the step and the separate calls give the
// same bits.
#include "dev_item.h"
#include "dev_summary.h"
#include "ls_flow.h"

namespace ls {

namespace {

constexpr int NW = kFlowWaves;
constexpr int NT = kFlowThreads;
constexpr int kMergeBatch = 4;   // split states the merger loads per round

// The ranker keeps a copy of the pair's page-table row in LDS when it fits.
template <int MAXC>
constexpr bool kPgLds = MAXC <= 2048;

template <int D, int MAXC>
struct FlowLds {
  int pg[kFlowMaxChunkBlocks];                      // score item: the chunk's page ids
  int ent[kFlowMaxSplit + item_entry_pad<NW>()];    // attention item: walk entries
  float red[2][NW];                                 // ranker: score range per wave
  int flag;
  union {
    struct {
      alignas(16) uint32_t stage[NW * 2 * 16 * Stage<D>::kKRowWords];
      float range[2 * NW];
    } s;
    struct {
      alignas(16) float sc[MAXC + MAXC / 16];       // padded score row
      TopkLds tk;
      TopkFastLds<> tf[MAXC <= kTopkFastMaxBlocks ? 1 : 0];
      int pgrow[kPgLds<MAXC> ? MAXC : 1];           // the pair's page-table row
    } t;
    ItemAttnLds<D, NW> at;
  } u;
};

__device__ __forceinline__ void flow_error(const FlowArgs& f) {
  st_dev(f.ctl + kCtlError, 1u);
}

// Counts one arrival at *ctr (device scope); true for the n-th, which also
// resets the counter. Called by one thread, after the caller's hand-off
// stores have completed.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, int n) {
  const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool last = prev == (uint32_t)(n - 1);
  if (last) st_dev(ctr, 0u);
  return last;
}

// Block-wide "any": one barrier.
__device__ __forceinline__ bool block_any(bool v) { return __syncthreads_or(v ? 1 : 0) != 0; }

// Walk entry of block blk of a request (page * 32 + valid tokens), or -1.
__device__ __forceinline__ int walk_entry(int blk, int page, const ReqGeom& geo, int num_pages) {
  if (blk < 0 || blk >= geo.nb) return -1;
  const int nt = geo.L - blk * 16 < 16 ? geo.L - blk * 16 : 16;
  return (page >= 0 && page < num_pages && nt > 0) ? page * 32 + nt : -1;
}

// Chunk c of pair `pair`: score its candidates into the key row; the pair's
// last chunk ranks the pair.
template <int D, int MAXC, bool kBounds, bool kAttn>
__device__ void flow_score(const FlowArgs& f, int item, FlowLds<D, MAXC>& sh) {
  const ScoreArgs& sa = f.sa;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int pair = item / f.chunks, c = item - pair * f.chunks;
  const int r = pair / sa.num_kv_heads, g = pair - r * sa.num_kv_heads;
  const ReqGeom geo = req_geom(sa.b, r, sa.n_sink, sa.n_recent);
  // the chunk: tiles [tb, tb + chunk_tiles) of the candidate range
  const int tb = geo.c0 / 16 + c * f.chunk_tiles;
  ReqGeom cg = geo;
  cg.c0 = geo.c0 > 16 * tb ? geo.c0 : 16 * tb;
  cg.c1 = geo.c1 < 16 * (tb + f.chunk_tiles) ? geo.c1 : 16 * (tb + f.chunk_tiles);
  if (cg.c1 < cg.c0) cg.c1 = cg.c0;
  const int n = cg.c1 - cg.c0;   // <= kFlowMaxChunkBlocks
  for (int i = tid; i < n; i += NT) sh.pg[i] = sa.b.indices[geo.page_base + cg.c0 + i];
  __syncthreads();
  uint32_t* row = f.keys + (size_t)pair * sa.b.max_blocks;
  if (n > 0) {
    float* rowf = reinterpret_cast<float*>(row);
    if constexpr (kBounds)
      item_score_bounds<D, MAXC, kStoreDevKey, NW>(sa, r, g, cg, sh.pg, rowf, sh.u.s.stage,
                                                   nullptr, cg.c0);
    else
      item_score<D, MAXC, kStoreDevKey, NW>(sa, r, g, cg, sh.pg, rowf, sh.u.s.stage, nullptr,
                                            cg.c0);
  }
  wait_stores();   // this thread's keys have reached the device-coherent level
  __syncthreads();   // (and every wave is done with the scoring tiles: the LDS is reused)
  if (tid == 0) sh.flag = arrive_last(f.ctl + kFlowCtlWords + (size_t)pair * 2, f.chunks);
  __syncthreads();
  if (!sh.flag) return;

  // ---- the ranker (last chunk to arrive): the key row, then the top-k ----
  // (raised wave priority: the ranking is on the pair's critical path, the
  // streaming workgroups sharing the CU are not)
  __builtin_amdgcn_s_setprio(3);
  const int nc = geo.c1 - geo.c0;
  constexpr int NPT = MAXC / NT;
  uint32_t kv[NPT];
#pragma unroll
  for (int m = 0; m < NPT; ++m) kv[m] = 0u;
  // the page-table row first: it does not depend on the scores
  if constexpr (kAttn && kPgLds<MAXC>) {
    int pv[NPT];
#pragma unroll
    for (int m = 0; m < NPT; ++m) {
      const int e = tid + m * NT;
      pv[m] = e < geo.nb ? sa.b.indices[geo.page_base + e] : 0;
    }
#pragma unroll
    for (int m = 0; m < NPT; ++m) {
      const int e = tid + m * NT;
      if (e < geo.nb) sh.u.t.pgrow[e] = pv[m];
    }
  }
#pragma unroll
  for (int m = 0; m < NPT; ++m) {   // every load issued before the uses
    const int e = tid + m * NT;
    if (e < nc) kv[m] = ld_dev(&row[geo.c0 + e]);
  }
  // decode, stage the row for the ranking, leave the key row zero
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int e = tid + m * NT;
    if (e < nc) {
      const uint32_t k = kv[m];
      const float v = __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
      sh.u.t.sc[e + (e >> 4)] = v;
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
      st_dev(&row[geo.c0 + e], 0u);
      if (f.scores_out) f.scores_out[(size_t)pair * sa.b.max_blocks + geo.c0 + e] = v;
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
  for (int w = 0; w < NW; ++w) {
    mn = fminf(mn, sh.red[0][w]);
    mx = fmaxf(mx, sh.red[1][w]);
  }
  const TopkArgs& ta = f.ta;
  int32_t* sel = ta.selected + (size_t)pair * ta.max_selected;
  int32_t* ent = kAttn ? f.ents + (size_t)pair * ta.max_selected : nullptr;
  const int32_t* pages = sa.b.indices + geo.page_base;
  const int num_pages = sa.b.num_pages;
  auto emit = [&](int p, int b) {
    sel[p] = b;
    if constexpr (kAttn) {
      int page = -1;
      if (b >= 0 && b < geo.nb) page = kPgLds<MAXC> ? sh.u.t.pgrow[b] : pages[b];
      st_dev(&ent[p], walk_entry(b, page, geo, num_pages));
    }
  };
  int stored;
  if constexpr (MAXC <= kTopkFastMaxBlocks) {
    stored = topk_fast<NPT, NT>(sh.u.t.sc, geo, topk_budget(ta, geo), ta.max_selected,
                                sh.u.t.tf[0], sh.u.t.tk, sel, ta.selected_count + pair, mn, mx,
                                emit);
  } else {
    // longer rows: the general workgroup top-k, read back for the entries
    stored = topk_wg<NPT, NT, true, true>(sh.u.t.sc, geo, topk_budget(ta, geo), sel,
                                          ta.max_selected, ta.selected_count + pair, sh.u.t.tk);
    if constexpr (kAttn) {
      wait_stores();
      __syncthreads();
      for (int p = tid; p < ta.max_selected; p += NT) emit(p, ld_dev(&sel[p]));
    }
  }
  if (tid == 0) ta.selected_count[pair] = stored;
  __builtin_amdgcn_s_setprio(0);
}

// Merge of the pair's split states in split order (online log-sum-exp),
// by the pair's last split to arrive: kMergeBatch states per round of
// loads, each word reset to zero once read.
template <int D>
__device__ void flow_merge(const FlowArgs& f, int r, int g) {
  const AttnArgs& a = f.aa;
  const int tid = threadIdx.x;
  constexpr int EPT = (4 * D + NT - 1) / NT;
  const int S = f.splits;
  float M[EPT], O[EPT], L[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    M[j] = kNegInf;
    O[j] = 0.0f;
    L[j] = 0.0f;
  }
  for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
    float wo[kMergeBatch][EPT], wm[kMergeBatch][EPT], wl[kMergeBatch][EPT];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {   // every load issued before the uses
      const int s = s0 + u;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int e = tid + j * NT;
        wo[u][j] = 0.0f;
        wm[u][j] = kNegInf;
        wl[u][j] = 0.0f;
        if (s < S && e < 4 * D) {
          const int h = e / D, d = e - h * D;
          const float* ph = reinterpret_cast<const float*>(f.parts) +
                            (((size_t)r * a.num_q_heads + g * 4 + h) * S + s) * (D + 2);
          wo[u][j] = ld_dev(ph + d);
          wm[u][j] = ld_dev(ph + D);
          wl[u][j] = ld_dev(ph + D + 1);
        }
      }
    }
    __syncthreads();   // every thread of a head has read its (m, l) words
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int e = tid + j * NT;
        if (s < S && e < 4 * D) {
          const int h = e / D, d = e - h * D;
          uint32_t* ph = f.parts + (((size_t)r * a.num_q_heads + g * 4 + h) * S + s) * (D + 2);
          st_dev(ph + d, 0u);
          if (d == 0) {
            st_dev(ph + D, 0u);
            st_dev(ph + D + 1, 0u);
          }
          const float Mn = fmaxf(M[j], wm[u][j]);
          if (Mn != kNegInf) {
            const float fa = exp2_fast(M[j] - Mn), fb = exp2_fast(wm[u][j] - Mn);   // -inf -> 0
            O[j] = O[j] * fa + wo[u][j] * fb;
            L[j] = L[j] * fa + wl[u][j] * fb;
            M[j] = Mn;
          }
        }
      }
    }
  }
  const bool out32 = a.out_dtype == LS_DTYPE_FP32;
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
}

// Split s of pair `pair`: its walk entries (polled in the step, built from
// the given selection otherwise), the attention, the state; the pair's last
// split merges.
template <int D, int MAXC, bool kScore>
__device__ void flow_attn(const FlowArgs& f, int item, FlowLds<D, MAXC>& sh) {
  const AttnArgs& a = f.aa;
  const int tid = threadIdx.x;
  const int pair = item / f.splits, s = item - pair * f.splits;
  const int r = pair / a.num_kv_heads, g = pair - r * a.num_kv_heads;
  const int p0 = s * f.split;
  int npos = a.max_selected - p0;   // positions of this split
  npos = npos < 0 ? 0 : (npos > f.split ? f.split : npos);
  if constexpr (kScore) {
    int32_t* erow = f.ents + (size_t)pair * a.max_selected + p0;
    int e = 0;
    for (int spins = 0;; ++spins) {
      if (tid < npos && e == 0) e = ld_dev(&erow[tid]);
      if (!block_any(tid < npos && e == 0)) break;
      if (spins >= kFlowSpinLimit) {
        if (tid == 0) flow_error(f);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (tid < npos) st_dev(&erow[tid], 0);
    // this thread's entry (tid < npos), then the padding item_attn may read
    for (int pos = tid; pos < item_entry_count<NW>(npos); pos += NT)
      sh.ent[pos] = (pos < npos && e != 0) ? e : -1;
  } else {
    const ReqGeom geo = req_geom(a.b, r, 0, 0);
    int total = a.selected_count[pair];
    total = total < 0 ? 0 : (total > a.max_selected ? a.max_selected : total);
    const int32_t* srow = a.selected + (size_t)pair * a.max_selected + p0;
    const int32_t* pages = a.b.indices + geo.page_base;
    for (int pos = tid; pos < item_entry_count<NW>(npos); pos += NT) {
      int e = -1;
      if (pos < npos && p0 + pos < total) {
        const int blk = srow[pos];
        e = walk_entry(blk, blk >= 0 && blk < geo.nb ? pages[blk] : -1, geo, a.b.num_pages);
      }
      sh.ent[pos] = e;
    }
  }
  __syncthreads();
  const ItemSplit sp{reinterpret_cast<float*>(f.parts), f.splits, s};
  item_attn<D, false, NW, kSplitDev, 1>(a, r, g, sh.ent, npos, sh.u.at, nullptr, &sp);
  wait_stores();   // this thread's state words have reached the device-coherent level
  __syncthreads();
  if (tid == 0)
    sh.flag = arrive_last(f.ctl + kFlowCtlWords + (size_t)pair * 2 + 1, f.splits);
  __syncthreads();
  if (!sh.flag) return;
  __builtin_amdgcn_s_setprio(3);
  flow_merge<D>(f, r, g);
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int MAXC, bool kBounds, bool kScore, bool kAttn>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(MAXC <= 4096 ? 4 : 2))) void flow_kernel(FlowArgs f) {
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

__global__ void zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
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

hipError_t launch_zero(void* p, size_t n, hipStream_t st) {
  const size_t words = n / sizeof(uint32_t);
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  blocks = blocks > 4096 ? 4096 : blocks;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace ls

// Per-(request, kv head) kernels: one 1024-thread workgroup per pair, grid
// (num_kv_heads, batch). See dev_item.h for the method and the memory walk.
//  * select_item_kernel: scoring + top-k (ls_score_select),
//  * attn_item_kernel:   attention over a given selection (ls_sparse_attn_decode),
//  * step_item_kernel:   the whole decode step of the pair (ls_sparse_decode_step);
//    the selection goes to the caller's buffers and stays in LDS for the
//    attention, so the step is one launch with no hand-off between workgroups.
#include "dev_item.h"
#include "dev_summary.h"

namespace ls {

// kBounds: the summaries are Quest bounds, scored by item_score_bounds.
template <int D, int MAXC, bool kBounds>
__global__ __launch_bounds__(kItemThreads) void select_item_kernel(ScoreArgs sa, TopkArgs ta) {
  __shared__ int pg[MAXC];
  __shared__ __attribute__((aligned(16))) float sc[MAXC];
  __shared__ TopkLds tk;
  __shared__ float range[2 * kItemWaves];
  __shared__ __attribute__((aligned(16))) uint32_t stage[kItemWaves * 2 * 16 * Stage<D>::kKRowWords];
  const int g = blockIdx.x, r = blockIdx.y;
  const int item = r * sa.num_kv_heads + g;
  const ReqGeom geo = req_geom(sa.b, r, sa.n_sink, sa.n_recent);
  load_page_row<MAXC>(sa.b, geo, pg);
  __syncthreads();
  if constexpr (kBounds) item_score_bounds<D, MAXC>(sa, r, g, geo, pg, sc, stage, range);
  else item_score<D, MAXC>(sa, r, g, geo, pg, sc, stage, range);
  __syncthreads();
  if (sa.scores) {
    float* out = sa.scores + (size_t)item * sa.b.max_blocks;
    for (int b = geo.c0 + threadIdx.x; b < geo.c1; b += kItemThreads) out[b] = sc[b];
  }
  (void)topk_wg<MAXC / kItemThreads, kItemThreads>(
      sc + geo.c0, geo, topk_budget(ta, geo), ta.selected + (size_t)item * ta.max_selected,
      ta.max_selected, ta.selected_count + item, tk, nullptr, range, kItemWaves);
}

template <int D, int MAXC>
__global__ __launch_bounds__(kItemThreads) void attn_item_kernel(AttnArgs a) {
  __shared__ int pg[MAXC];
  __shared__ int sel[MAXC + kItemEntryPad];
  __shared__ ItemAttnLds<D> sh;
  const int g = blockIdx.x, r = blockIdx.y;
  const size_t item = (size_t)r * a.num_kv_heads + g;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  load_page_row<MAXC>(a.b, geo, pg);
  int cnt;
  if (a.selected) {
    // the count and the entries in one hop; entries past the count are unused
    cnt = a.selected_count[item];
    const int n = a.max_selected < MAXC ? a.max_selected : MAXC;
    const int32_t* row = a.selected + item * a.max_selected;
    for (int i = threadIdx.x; i < n; i += kItemThreads) sel[i] = row[i];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
  } else {
    cnt = geo.nb;
    for (int i = threadIdx.x; i < geo.nb; i += kItemThreads) sel[i] = i;
  }
  __syncthreads();
  item_entries(a, geo, sel, cnt, pg, item_entry_count(cnt));
  __syncthreads();
  item_attn<D>(a, r, g, sel, cnt, sh);
}

// Rows of the grid past the batch refresh the summaries of the pages that
// just filled (one wave per (page, head) tile), concurrently with the pairs'
// steps: those pages are not scored in this call (the caller guarantees it).
template <int D, int MAXC, bool kBounds>
__global__ __launch_bounds__(kItemThreads) void step_item_kernel(ScoreArgs sa, TopkArgs ta,
                                                                 AttnArgs aa, SummaryUpdate up) {
  if ((int)blockIdx.y >= sa.b.batch) {
    const int tile = ((blockIdx.y - sa.b.batch) * gridDim.x + blockIdx.x) * kItemWaves + wave_id();
    if (tile < up.n_tiles) {
      if constexpr (kBounds)
        bounds_tile_bf16<D>(up.keys, up.pages, tile, sa.b.num_pages, sa.num_kv_heads,
                            sa.b.page_size, static_cast<uint16_t*>(up.out));
      else
        summary_tile_bf16<D, false>(up.keys, up.pages, tile, sa.b.num_pages, sa.num_kv_heads,
                                    sa.b.page_size, up.out);
    }
    return;
  }
  __shared__ int pg[MAXC];
  __shared__ int sel[MAXC + kItemEntryPad];
  __shared__ union {
    struct {
      alignas(16) float sc[MAXC];
      TopkLds tk;
      float range[2 * kItemWaves];
      alignas(16) uint32_t stage[kItemWaves * 2 * 16 * Stage<D>::kKRowWords];
    } s;
    ItemAttnLds<D> at;
  } u;
  const int g = blockIdx.x, r = blockIdx.y;
  const int item = r * sa.num_kv_heads + g;
  const ReqGeom geo = req_geom(sa.b, r, sa.n_sink, sa.n_recent);
  load_page_row<MAXC>(sa.b, geo, pg);
  __syncthreads();
  if constexpr (kBounds) item_score_bounds<D, MAXC>(sa, r, g, geo, pg, u.s.sc, u.s.stage, u.s.range);
  else item_score<D, MAXC>(sa, r, g, geo, pg, u.s.sc, u.s.stage, u.s.range);
  __syncthreads();
  const int cnt = topk_wg<MAXC / kItemThreads, kItemThreads>(
      u.s.sc + geo.c0, geo, topk_budget(ta, geo), ta.selected + (size_t)item * ta.max_selected,
      ta.max_selected, ta.selected_count + item, u.s.tk, sel, u.s.range, kItemWaves);
  item_entries(aa, geo, sel, cnt, pg, item_entry_count(cnt));
  __syncthreads();
  item_attn<D>(aa, r, g, sel, cnt, u.at);
}

// ---------------------------------------------------------------------------
// Two workgroups per pair (batches with at most kPairMaxPairs pairs, so that
// the grid still covers the chip): the scoring is split over the pair's two
// workgroups (score_part_kernel, scores through HBM), then both workgroups
// rank the same scores (identical selections), each attends every other group
// of 8 selection positions, and the second to finish merges the two softmax
// states (arrival counter, no waiting).

// Scores of half `blockIdx.x` of the candidate tiles of pair (r, g) into the
// score row; also zeroes the pair's arrival counter for the attention launch.
template <int D, int MAXC>
__global__ __launch_bounds__(kItemThreads) void score_part_kernel(ScoreArgs sa, float* scores,
                                                                  uint32_t* arrivals) {
  __shared__ int pg[MAXC];
  __shared__ __attribute__((aligned(16))) uint32_t stage[kItemWaves * 2 * 16 * Stage<D>::kKRowWords];
  const int part = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int item = r * sa.num_kv_heads + g;
  if (part == 0 && threadIdx.x == 0) arrivals[item] = 0u;
  ReqGeom geo = req_geom(sa.b, r, sa.n_sink, sa.n_recent);
  const int t0 = geo.c0 / 16, t1 = (geo.c1 + 15) / 16;
  const int half = (t1 - t0 + 1) / 2;
  const int lo = (t0 + part * half) * 16, hi = (t0 + (part + 1) * half) * 16;
  geo.c0 = geo.c0 > lo ? geo.c0 : lo;
  geo.c1 = geo.c1 < hi ? geo.c1 : hi;
  if (geo.c1 <= geo.c0) return;
  for (int b = geo.c0 + threadIdx.x; b < geo.c1; b += kItemThreads)
    pg[b] = sa.b.indices[geo.page_base + b];
  __syncthreads();
  item_score<D, MAXC, kStoreGlobal>(sa, r, g, geo, pg, scores + (size_t)item * sa.b.max_blocks, stage);
}

template <int D, int MAXC>
__global__ __launch_bounds__(kItemThreads) void select_attn_pair_kernel(TopkArgs ta, AttnArgs aa,
                                                                        float* pair_part,
                                                                        uint32_t* arrivals) {
  __shared__ int pg[MAXC];
  __shared__ int sel[MAXC + kItemEntryPad];
  __shared__ union {
    struct {
      alignas(16) float sc[MAXC];
      TopkLds tk;
    } s;
    ItemAttnLds<D> at;
  } u;
  const int half = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int item = r * ta.num_kv_heads + g;
  const ReqGeom geo = req_geom(ta.b, r, ta.n_sink, ta.n_recent);
  load_page_row<MAXC>(ta.b, geo, pg);
  const float* srow = ta.scores + (size_t)item * ta.b.max_blocks;
  {
    constexpr int NPT = MAXC / kItemThreads;   // every load issued before the stores
    float v[NPT];
#pragma unroll
    for (int m = 0; m < NPT; ++m) {
      const int b = geo.c0 + threadIdx.x + m * kItemThreads;
      v[m] = b < geo.c1 ? srow[b] : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < NPT; ++m) {
      const int b = geo.c0 + threadIdx.x + m * kItemThreads;
      if (b < geo.c1) u.s.sc[b] = v[m];
    }
  }
  __syncthreads();
  const int cnt = topk_wg<MAXC / kItemThreads, kItemThreads>(
      u.s.sc + geo.c0, geo, topk_budget(ta, geo), ta.selected + (size_t)item * ta.max_selected,
      ta.max_selected, ta.selected_count + item, u.s.tk, sel);
  item_entries(aa, geo, sel, cnt, pg, item_entry_count(cnt));
  __syncthreads();
  const ItemPair pr{pair_part + (size_t)item * kPairFloats<D>, arrivals + item, half};
  item_attn<D>(aa, r, g, sel, cnt, u.at, &pr);
}

__global__ void pair_zero_kernel(uint32_t* arrivals, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) arrivals[i] = 0u;
}

template <int D, int MAXC>
__global__ __launch_bounds__(kItemThreads) void attn_pair_kernel(AttnArgs a, float* pair_part,
                                                                 uint32_t* arrivals) {
  __shared__ int pg[MAXC];
  __shared__ int sel[MAXC + kItemEntryPad];
  __shared__ ItemAttnLds<D> sh;
  const int half = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const size_t item = (size_t)r * a.num_kv_heads + g;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  load_page_row<MAXC>(a.b, geo, pg);
  int cnt;
  if (a.selected) {
    cnt = a.selected_count[item];
    const int n = a.max_selected < MAXC ? a.max_selected : MAXC;
    const int32_t* row = a.selected + item * a.max_selected;
    for (int i = threadIdx.x; i < n; i += kItemThreads) sel[i] = row[i];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
  } else {
    cnt = geo.nb;
    for (int i = threadIdx.x; i < geo.nb; i += kItemThreads) sel[i] = i;
  }
  __syncthreads();
  item_entries(a, geo, sel, cnt, pg, item_entry_count(cnt));
  __syncthreads();
  const ItemPair pr{pair_part + item * kPairFloats<D>, arrivals + item, half};
  item_attn<D>(a, r, g, sel, cnt, sh, &pr);
}

// Split s of pair (r, g): positions [s * chunk, s * chunk + chunk) of the
// pair's selection row (of its block list when there is no selection), read
// straight from the page table into walk entries, attended by the eight
// waves and written as split s of the partials.
template <int D>
__global__ __launch_bounds__(kItemThreads) void attn_chunk_kernel(AttnArgs a, int chunk) {
  __shared__ int ent[kChunkMaxBlocks + kItemEntryPad];
  __shared__ ItemAttnLds<D> sh;
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const size_t item = (size_t)r * a.num_kv_heads + g;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const bool sparse = a.selected != nullptr;
  int total = geo.nb;
  if (sparse) {
    total = a.selected_count[item];
    total = total < 0 ? 0 : (total > a.max_selected ? a.max_selected : total);
  }
  const int p0 = s * chunk;
  int cnt = total - p0;
  cnt = cnt < 0 ? 0 : (cnt > chunk ? chunk : cnt);
  const int32_t* pages = a.b.indices + geo.page_base;
  const int32_t* row = sparse ? a.selected + item * a.max_selected + p0 : nullptr;
  for (int pos = threadIdx.x; pos < item_entry_count(cnt); pos += kItemThreads) {
    int e = -1;
    if (pos < cnt) {
      const int blk = sparse ? row[pos] : p0 + pos;
      if (blk >= 0 && blk < geo.nb) {
        const int p = pages[blk];
        const int nt = geo.L - blk * 16 < 16 ? geo.L - blk * 16 : 16;
        if (p >= 0 && p < a.b.num_pages && nt > 0) e = p * 32 + nt;
      }
    }
    ent[pos] = e;
  }
  __syncthreads();
  const ItemSplit sp{a.partials, a.num_splits, s};
  item_attn<D>(a, r, g, ent, cnt, sh, nullptr, &sp);
}

// Split s of pair (r, g) of the sink + recent window: the pair's positions
// are the sink blocks (tokens [0, ns), ns = min(win_sink, L)) then the
// window blocks (tokens [lo, L), lo = max(ns, L - win_len)); when lo = ns the
// two ranges touch and the positions are simply the request's blocks. A
// block holding both the last sinks and the first window tokens appears
// twice, with disjoint token ranges. Walk entries carry the first valid
// token (item_attn's kLo form).
template <int D>
__global__ __launch_bounds__(kItemThreads) void attn_window_kernel(AttnArgs a, int chunk) {
  __shared__ int ent[kChunkMaxBlocks + kItemEntryPad];
  __shared__ ItemAttnLds<D> sh;
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const int L = geo.L;
  const int ns = a.win_sink < L ? a.win_sink : L;
  const int lw = L - a.win_len;
  const int lo = lw > ns ? lw : ns;
  const bool gap = lo > ns;
  const int nsb = gap ? (ns + 15) / 16 : 0;          // sink positions
  const int wb0 = gap ? lo / 16 : 0;                  // first window block
  const int t_lo = gap ? lo : 0;                      // first window token (all tokens: 0)
  const int total = nsb + (geo.nb - wb0 > 0 ? geo.nb - wb0 : 0);
  const int p0 = s * chunk;
  int cnt = total - p0;
  cnt = cnt < 0 ? 0 : (cnt > chunk ? chunk : cnt);
  const int32_t* pages = a.b.indices + geo.page_base;
  for (int pos = threadIdx.x; pos < item_entry_count(cnt); pos += kItemThreads) {
    int e = -1;
    if (pos < cnt) {
      const int q = p0 + pos;
      int blk, t0, t1;   // tokens [t0, t1) of block blk
      if (q < nsb) {
        blk = q;
        t0 = 16 * blk;
        t1 = ns < 16 * blk + 16 ? ns : 16 * blk + 16;
      } else {
        blk = wb0 + (q - nsb);
        t0 = t_lo > 16 * blk ? t_lo : 16 * blk;
        t1 = L < 16 * blk + 16 ? L : 16 * blk + 16;
      }
      if (blk >= 0 && blk < geo.nb && t1 > t0) {
        const int p = pages[blk];
        if (p >= 0 && p < a.b.num_pages) e = p * 512 + (t0 - 16 * blk) * 32 + (t1 - 16 * blk);
      }
    }
    ent[pos] = e;
  }
  __syncthreads();
  const ItemSplit sp{a.partials, a.num_splits, s};
  item_attn<D, true>(a, r, g, ent, cnt, sh, nullptr, &sp);
}

hipError_t launch_attn_window(const AttnArgs& a0, int max_pos, hipStream_t st) {
  AttnArgs a = a0;
  const int n = max_pos < 1 ? 1 : max_pos;
  const int pairs = a.b.batch * a.num_kv_heads;
  constexpr int kTargetWgs = 512;   // two per CU: windows are short, longer runs ramp less
  int splits = (kTargetWgs + pairs - 1) / pairs;
  const int most = (n + 15) / 16;
  splits = splits > most ? most : splits;
  splits = splits < 1 ? 1 : splits;
  int chunk = (n + splits - 1) / splits;
  chunk = (chunk + kAttnBlocksPerSplit - 1) / kAttnBlocksPerSplit * kAttnBlocksPerSplit;
  chunk = chunk > kChunkMaxBlocks ? kChunkMaxBlocks : chunk;
  chunk = chunk < kAttnBlocksPerSplit ? kAttnBlocksPerSplit : chunk;
  a.num_splits = (n + chunk - 1) / chunk;
  if (a.num_splits < 1) a.num_splits = 1;
  if (a.num_splits > a0.num_splits) return hipErrorInvalidValue;   // partials capacity
  const dim3 grid(a.num_splits, a.num_kv_heads, a.b.batch);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((attn_window_kernel<128>), grid, dim3(kItemThreads), 0, st, a, chunk);
  else
    hipLaunchKernelGGL((attn_window_kernel<64>), grid, dim3(kItemThreads), 0, st, a, chunk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(a, st);
}

bool pair_path(int batch, int hkv, int max_blocks) {
  return (long long)batch * hkv <= kPairMaxPairs && max_blocks > kPairMinBlocks;
}

bool item_path(int batch, int hkv, int head_dim, int group, int max_blocks, int num_pages) {
  return (long long)batch * hkv >= kItemMinPairs && group == 4 &&
         (head_dim == 128 || head_dim == 64) && max_blocks <= 8192 && num_pages < (1 << 26);
}

#define LS_ITEM_DISPATCH(LAUNCH)                      \
  if (D == 128) {                                     \
    if (n <= 1024) LAUNCH(128, 1024);                 \
    if (n <= 2048) LAUNCH(128, 2048);                 \
    if (n <= 4096) LAUNCH(128, 4096);                 \
    LAUNCH(128, 8192);                                \
  }                                                   \
  if (n <= 1024) LAUNCH(64, 1024);                    \
  if (n <= 2048) LAUNCH(64, 2048);                    \
  if (n <= 4096) LAUNCH(64, 4096);                    \
  LAUNCH(64, 8192);

hipError_t launch_select_item(const ScoreArgs& sa, const TopkArgs& ta, hipStream_t st) {
  const int D = sa.head_dim, n = sa.b.max_blocks;
  const dim3 grid(sa.num_kv_heads, sa.b.batch);
#define LAUNCH(DD, MC)                                                                    \
  do {                                                                                    \
    if (sa.bounds)                                                                        \
      hipLaunchKernelGGL((select_item_kernel<DD, MC, true>), grid, dim3(kItemThreads), 0, \
                         st, sa, ta);                                                     \
    else                                                                                  \
      hipLaunchKernelGGL((select_item_kernel<DD, MC, false>), grid, dim3(kItemThreads), 0, \
                         st, sa, ta);                                                     \
    return hipGetLastError();                                                             \
  } while (0)
  LS_ITEM_DISPATCH(LAUNCH)
#undef LAUNCH
}

hipError_t launch_attn_item(const AttnArgs& a, hipStream_t st) {
  const int D = a.head_dim, n = a.b.max_blocks;
  if (pair_path(a.b.batch, a.num_kv_heads, n)) {
    const int pairs = a.b.batch * a.num_kv_heads;
    float* part = a.partials;
    uint32_t* arr = pair_arrivals(a.partials, pairs, D);
    hipLaunchKernelGGL(pair_zero_kernel, dim3((pairs + 255) / 256), dim3(256), 0, st, arr, pairs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid2(2, a.num_kv_heads, a.b.batch);
#define LAUNCH(DD, MC)                                                                    \
  do {                                                                                    \
    hipLaunchKernelGGL((attn_pair_kernel<DD, MC>), grid2, dim3(kItemThreads), 0, st, a, part, \
                       arr);                                                              \
    return hipGetLastError();                                                             \
  } while (0)
    LS_ITEM_DISPATCH(LAUNCH)
#undef LAUNCH
  }
  const dim3 grid(a.num_kv_heads, a.b.batch);
#define LAUNCH(DD, MC)                                                                  \
  do {                                                                                  \
    hipLaunchKernelGGL((attn_item_kernel<DD, MC>), grid, dim3(kItemThreads), 0, st, a); \
    return hipGetLastError();                                                           \
  } while (0)
  LS_ITEM_DISPATCH(LAUNCH)
#undef LAUNCH
}

hipError_t launch_attn_chunked(const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  const int n = a.selected ? a.max_selected : a.b.max_blocks;   // positions per pair
  const int pairs = a.b.batch * a.num_kv_heads;
  // about 2048 workgroups (8 per CU), at least 16 positions (two per wave)
  // per split and at most kChunkMaxBlocks; pairs of at most 1024 positions
  // take about 512 (longer runs ramp less)
  const int kTargetWgs = n <= 1024 ? 512 : 2048;
  int splits = (kTargetWgs + pairs - 1) / pairs;
  const int most = (n + 15) / 16;
  splits = splits > most ? most : splits;
  splits = splits < 1 ? 1 : splits;
  int chunk = (n + splits - 1) / splits;
  chunk = (chunk + kAttnBlocksPerSplit - 1) / kAttnBlocksPerSplit * kAttnBlocksPerSplit;
  chunk = chunk > kChunkMaxBlocks ? kChunkMaxBlocks : chunk;
  chunk = chunk < kAttnBlocksPerSplit ? kAttnBlocksPerSplit : chunk;
  a.num_splits = (n + chunk - 1) / chunk;
  if (a.num_splits < 1) a.num_splits = 1;
  if (a.num_splits > a0.num_splits) return hipErrorInvalidValue;   // partials capacity
  const dim3 grid(a.num_splits, a.num_kv_heads, a.b.batch);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((attn_chunk_kernel<128>), grid, dim3(kItemThreads), 0, st, a, chunk);
  else
    hipLaunchKernelGGL((attn_chunk_kernel<64>), grid, dim3(kItemThreads), 0, st, a, chunk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(a, st);
}

hipError_t launch_step_item(const ScoreArgs& sa, const TopkArgs& ta, const AttnArgs& aa,
                            const SummaryUpdate& up, hipStream_t st) {
  const int D = sa.head_dim, n = sa.b.max_blocks;
  const bool one_launch = !pair_path(sa.b.batch, sa.num_kv_heads, n) && n <= 4096;
  if (sa.bounds && pair_path(sa.b.batch, sa.num_kv_heads, n))
    return hipErrorInvalidValue;   // no two-workgroup scoring of bounds (checked by the caller)
  if (up.n_tiles > 0 && !one_launch) {
    // the multi-launch forms refresh the summaries first
    SummaryArgs su{up.keys, nullptr, ls_pool{sa.b.num_pages, sa.num_kv_heads, sa.b.page_size, D,
                                             LS_DTYPE_BF16},
                   up.pages, up.n_tiles / sa.num_kv_heads, up.out, LS_DTYPE_BF16};
    const hipError_t e = sa.bounds ? launch_bounds(su, st) : launch_summaries(su, st);
    if (e != hipSuccess) return e;
  }
  if (pair_path(sa.b.batch, sa.num_kv_heads, n)) {
    // scoring over both workgroups of each pair, then top-k + attention
    const int pairs = sa.b.batch * sa.num_kv_heads;
    float* part = aa.partials;
    uint32_t* arr = pair_arrivals(aa.partials, pairs, D);
    const dim3 grid2(2, sa.num_kv_heads, sa.b.batch);
#define LAUNCH(DD, MC)                                                                       \
  do {                                                                                       \
    hipLaunchKernelGGL((score_part_kernel<DD, MC>), grid2, dim3(kItemThreads), 0, st, sa,      \
                       const_cast<float*>(ta.scores), arr);                                  \
    hipError_t e = hipGetLastError();                                                        \
    if (e != hipSuccess) return e;                                                           \
    hipLaunchKernelGGL((select_attn_pair_kernel<DD, MC>), grid2, dim3(kItemThreads), 0, st, ta, \
                       aa, part, arr);                                                       \
    return hipGetLastError();                                                                \
  } while (0)
    LS_ITEM_DISPATCH(LAUNCH)
#undef LAUNCH
  }
  if (n > 4096) {
    // the one-launch form does not fit in LDS: the two per-pair launches,
    // which are the separate calls (same results)
    const hipError_t e = launch_select_item(sa, ta, st);
    return e != hipSuccess ? e : launch_attn_item(aa, st);
  }
  const int per_row = kItemWaves * sa.num_kv_heads;   // update tiles per extra grid row
  const dim3 grid(sa.num_kv_heads, sa.b.batch + (up.n_tiles + per_row - 1) / per_row);
#define LAUNCH(DD, MC)                                                                      \
  do {                                                                                      \
    if (sa.bounds)                                                                          \
      hipLaunchKernelGGL((step_item_kernel<DD, MC, true>), grid, dim3(kItemThreads), 0, st, \
                         sa, ta, aa, up);                                                   \
    else                                                                                    \
      hipLaunchKernelGGL((step_item_kernel<DD, MC, false>), grid, dim3(kItemThreads), 0, st, \
                         sa, ta, aa, up);                                                   \
    return hipGetLastError();                                                               \
  } while (0)
  if (D == 128) {
    if (n <= 1024) LAUNCH(128, 1024);
    if (n <= 2048) LAUNCH(128, 2048);
    LAUNCH(128, 4096);
  }
  if (n <= 1024) LAUNCH(64, 1024);
  if (n <= 2048) LAUNCH(64, 2048);
  LAUNCH(64, 4096);
#undef LAUNCH
}

#undef LS_ITEM_DISPATCH

}  // namespace ls

// C ABI of libls: host-side validation, workspace sizing and kernel dispatch.
// Every entry point validates its arguments before touching HIP, enqueues on
// the caller's stream, never synchronises and never allocates device memory.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "ls_flow.h"
#include "ls_internal.h"
#include "ls_plan.h"

namespace {

thread_local char g_err[512] = "";

ls_status fail(ls_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ls_status ok() {
  g_err[0] = '\0';
  return LS_OK;
}

ls_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// The kernels read q, pools and summaries 16 bytes at a time.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

ls_status check_batch(const ls_batch& b) {
  if (b.batch_size < 0) return fail(LS_ERR_INVALID, "batch.batch_size < 0");
  if (b.batch_size == 0) return ok();
  if (!b.page_indptr || !b.page_indices || !b.seq_lens)
    return fail(LS_ERR_INVALID, "batch page_indptr / page_indices / seq_lens must be non-null");
  if (b.max_blocks < 1) return fail(LS_ERR_INVALID, "batch.max_blocks must be >= 1");
  return ok();
}

// GQA group sizes: 4 on every route (the matrix-core kernels tile 4 query
// heads x 16 tokens); 1, 2 and 8 on the split kernels, which take the group
// as a template parameter.
bool group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

ls_status check_gqa_pool(const ls_pool& p, const char* which) {
  if (p.num_pages < 1 || p.num_heads < 1)
    return fail(LS_ERR_INVALID, "%s: num_pages and num_heads must be >= 1", which);
  if (p.page_size != 16)
    return fail(LS_ERR_UNSUPPORTED, "%s: page_size %d (supported: 16)", which, p.page_size);
  if (p.head_dim != 64 && p.head_dim != 128)
    return fail(LS_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", which, p.head_dim);
  if (p.dtype != LS_DTYPE_BF16)
    return fail(LS_ERR_UNSUPPORTED, "%s: dtype %d (supported: bf16)", which, p.dtype);
  if (p.num_heads > 16 || !pow2(p.num_heads))
    return fail(LS_ERR_UNSUPPORTED, "%s: num_heads %d (supported: 1, 2, 4, 8, 16)", which,
                p.num_heads);
  return ok();
}

ls::BatchArgs batch_args(const ls_batch& b, const ls_pool& p) {
  ls::BatchArgs a;
  a.batch = b.batch_size;
  a.max_blocks = b.max_blocks;
  a.indptr = b.page_indptr;
  a.indices = b.page_indices;
  a.seq_lens = b.seq_lens;
  a.num_pages = p.num_pages;
  a.page_size = p.page_size;
  return a;
}

// ---- debug check of batches (ls_debug_enable, LS_DEBUG)

constexpr int kDebugMaxDevices = 64;

// Per GPU: kinds found (OR), calls with a violation, violating requests,
// calls checked. Zero when the library is loaded; ls_debug_report clears
// them. In host code the name is only a stand-in: the device address comes
// from hipGetSymbolAddress.
static __device__ __align__(16) int32_t debug_words[4];

std::mutex g_debug_mu;
void* g_debug_ptr[kDebugMaxDevices] = {};
std::atomic<int> g_debug{-1};   // -1: the environment not read yet

bool debug_on() {
  int v = g_debug.load();
  if (v < 0) {
    const char* e = std::getenv("LS_DEBUG");
    int expected = -1;
    g_debug.compare_exchange_strong(expected, (e && e[0] && std::strcmp(e, "0") != 0) ? 1 : 0);
    v = g_debug.load();
  }
  return v == 1;
}

// The calling thread's current device's copy of debug_words.
hipError_t debug_words_ptr(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDebugMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  if (!g_debug_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_words));
    if (e != hipSuccess) return e;
    g_debug_ptr[dev] = p;
  }
  *out = static_cast<int32_t*>(g_debug_ptr[dev]);
  return hipSuccess;
}

// In debug mode, the batch check ahead of a call's kernels, on its stream.
ls_status debug_check(const ls::BatchArgs& b, hipStream_t stream) {
  if (b.batch == 0 || !debug_on()) return ok();
  int32_t* words = nullptr;
  const hipError_t e = debug_words_ptr(&words);
  if (e != hipSuccess) return hip_status(e, "debug words address lookup");
  return hip_status(ls::launch_batch_check(b, words, true, stream), "batch check launch");
}

int max_total_selected(const ls_select_params& p, int max_blocks) {
  long long forced = (long long)p.n_sink + p.n_recent + 1;
  long long total;
  if (p.topk >= 0) {
    total = forced + p.topk;
  } else {
    long long byratio = (long long)std::ceil((double)p.keep_ratio * max_blocks) + 1;
    total = byratio > forced ? byratio : forced;
  }
  return (int)(total < max_blocks ? total : max_blocks);
}

ls::ScoreArgs score_args(const void* q, int num_q_heads, const void* summaries,
                         const ls_pool& pool, const ls_batch& batch, const ls_select_params& p,
                         float* scores) {
  ls::ScoreArgs sa;
  sa.q = static_cast<const uint16_t*>(q);
  sa.summaries = static_cast<const uint16_t*>(summaries);
  sa.b = batch_args(batch, pool);
  sa.num_q_heads = num_q_heads;
  sa.num_kv_heads = pool.num_heads;
  sa.head_dim = pool.head_dim;
  sa.group_agg = p.group_agg;
  sa.n_sink = p.n_sink;
  sa.n_recent = p.n_recent;
  sa.scores = scores;
  sa.bounds = p.score_mode == LS_SCORE_BOUNDS ? 1 : 0;
  return sa;
}

// Shapes the bounds scoring supports: the per-pair selection kernel (any
// number of pairs) with its walk-entry encoding.
bool bounds_ok(const ls_pool& pool, const ls_batch& batch) {
  return batch.max_blocks <= 8192 && pool.num_pages < (1 << 26);
}

ls::TopkArgs topk_args(const ls::ScoreArgs& sa, const ls_select_params& p, const float* scores,
                       int32_t* selected, int32_t* selected_count) {
  ls::TopkArgs ta;
  ta.scores = scores;
  ta.b = sa.b;
  ta.num_kv_heads = sa.num_kv_heads;
  ta.topk = p.topk;
  ta.keep_ratio = p.keep_ratio;
  ta.n_sink = p.n_sink;
  ta.n_recent = p.n_recent;
  ta.max_selected = p.max_selected;
  ta.selected = selected;
  ta.selected_count = selected_count;
  return ta;
}

ls::AttnArgs attn_args(const void* q, int num_q_heads, const void* k_pool, const void* v_pool,
                       const ls_pool& pool, const ls_batch& batch, const int32_t* selected,
                       const int32_t* selected_count, int max_selected, int num_splits,
                       float sm_scale, float* partials, void* out, int out_dtype, float* lse) {
  ls::AttnArgs aa;
  aa.q = static_cast<const uint16_t*>(q);
  aa.k_pool = static_cast<const uint16_t*>(k_pool);
  aa.v_pool = static_cast<const uint16_t*>(v_pool);
  aa.b = batch_args(batch, pool);
  aa.num_q_heads = num_q_heads;
  aa.num_kv_heads = pool.num_heads;
  aa.head_dim = pool.head_dim;
  aa.selected = selected;
  aa.selected_count = selected_count;
  aa.max_selected = max_selected;
  aa.num_splits = num_splits;
  aa.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  aa.partials = partials;
  aa.out = out;
  aa.out_dtype = out_dtype;
  aa.lse = lse;
  aa.win_sink = 0;
  aa.win_len = 0;
  return aa;
}

// ---- workspace layouts: the flow kernel's control words first (they must
// be zero before a workspace's first use, and every call leaves them zero),
// then the regions each path needs -------------------------------------------
// ---- workspace layouts. A workspace must be zero-filled before its first
// use and every call leaves it zero again: the flow kernel's hand-off words
// are zero until written and are reset by their readers; the split and
// dense paths zero what they wrote once their last kernel has run.
// [control words][block scores or keys][walk entries (step)][split states]
struct SelectWs {
  size_t rows, total;
};
SelectWs select_ws(int B, int hkv, int max_blocks) {
  SelectWs w;
  w.rows = ls::flow_ctl_bytes(B * hkv);
  w.total = w.rows + ls::flow_keys_bytes(B * hkv, max_blocks);
  return w;
}

// Split states of the attention: the split-K kernels', the flow kernel's
// and the planned kernels' (one slot pair per attention workgroup).
size_t attn_parts_bytes(int B, int hq, int head_dim, int max_selected, int max_blocks) {
  const int cap = max_selected > 0 ? max_selected : max_blocks;
  const size_t split = (size_t)B * hq * ls_attn_num_splits(cap) * (head_dim + 2) * sizeof(float);
  const int pairs = B * ((hq + 3) / 4);
  const size_t flow =
      ls::flow_parts_bytes(pairs, head_dim, ls::flow_plan(pairs, max_blocks, cap).splits);
  const size_t plan = ls::plan_slots_bytes(head_dim);
  return align_up(std::max(split, std::max(flow, plan)));
}

struct AttnWs {
  size_t parts, total;
};
// (counters for up to B * hq pairs: the size query does not know num_kv_heads)
AttnWs attn_ws(int B, int hq, int head_dim, int max_selected, int max_blocks) {
  AttnWs w;
  w.parts = ls::flow_ctl_bytes(B * hq);
  w.total = w.parts + attn_parts_bytes(B, hq, head_dim, max_selected, max_blocks);
  return w;
}

struct StepWs {
  size_t rows, ents, parts, total;
};
StepWs step_ws(int B, int hq, int hkv, int head_dim, int max_blocks, int max_selected) {
  StepWs w;
  w.rows = ls::flow_ctl_bytes(B * hkv);
  w.ents = w.rows + ls::flow_keys_bytes(B * hkv, max_blocks);
  w.parts = w.ents + ls::flow_ents_bytes(B * hkv, max_selected);
  w.total = w.parts + attn_parts_bytes(B, hq, head_dim, max_selected, max_blocks);
  return w;
}

// Which kernels serve a selection / attention / step call. The per-pair
// kernels (one workgroup owns a (request, kv head) pair from scoring to
// output, no hand-off between workgroups) are fastest when there are at
// least kItemMinPairs pairs of at most 4096 blocks. Longer requests in such
// batches take the planned kernels (work cut into equal ranges over all
// pairs, whatever their lengths). Fewer pairs take the flow kernel (a pair
// spread over many workgroups in one launch) up to kFlowMaxBlocks blocks,
// then the planned kernels; other shapes take the split kernels.
enum Route { kRouteItem, kRouteFlow, kRoutePlan, kRouteSplit };
Route route(const ls_pool& pool, const ls_batch& batch, int num_q_heads) {
  const int group = num_q_heads / pool.num_heads;
  const int pairs = batch.batch_size * pool.num_heads;
  if (ls::item_path(batch.batch_size, pool.num_heads, pool.head_dim, group, batch.max_blocks,
                    pool.num_pages) &&
      batch.max_blocks <= 4096)
    return kRouteItem;
  const bool plan = ls::plan_ok(group, pool.head_dim, batch.max_blocks, pool.num_pages, pairs);
  if (plan && pairs >= ls::kItemMinPairs) return kRoutePlan;
  if (ls::flow_ok(group, pool.head_dim, batch.max_blocks, pool.num_pages)) return kRouteFlow;
  if (plan) return kRoutePlan;
  return kRouteSplit;
}

ls::PlanArgs plan_args(const ls::ScoreArgs& sa, const ls::TopkArgs& ta, const ls::AttnArgs& aa,
                       const ls::SummaryUpdate& up, int pairs, int max_blocks, char* w,
                       size_t rows_off, size_t slots_off, float* scores_out,
                       size_t ents_off = 0) {
  ls::PlanArgs p;
  p.sa = sa;
  p.ta = ta;
  p.aa = aa;
  p.up = up;
  p.rows = scores_out ? scores_out : reinterpret_cast<float*>(w + rows_off);
  p.zero_rows = scores_out == nullptr;
  p.ta.scores = p.rows;
  p.ents = ents_off ? reinterpret_cast<int32_t*>(w + ents_off) : nullptr;
  p.ctl = reinterpret_cast<uint32_t*>(w);
  p.slots = reinterpret_cast<float*>(w + slots_off);
  p.pairs = pairs;
  p.max_blocks = max_blocks;
  return p;
}

ls::FlowArgs flow_args(const ls::ScoreArgs& sa, const ls::TopkArgs& ta, const ls::AttnArgs& aa,
                       const ls::SummaryUpdate& up, int pairs, int max_blocks, int max_selected,
                       char* w, size_t keys_off, size_t ents_off, size_t parts_off,
                       float* scores_out) {
  ls::FlowArgs f;
  f.sa = sa;
  f.ta = ta;
  f.aa = aa;
  f.up = up;
  f.ctl = reinterpret_cast<uint32_t*>(w);
  f.keys = reinterpret_cast<uint32_t*>(w + keys_off);
  f.ents = reinterpret_cast<int32_t*>(w + ents_off);
  f.parts = reinterpret_cast<uint32_t*>(w + parts_off);
  f.scores_out = scores_out;
  f.pairs = pairs;
  f.max_blocks = max_blocks;
  const ls::FlowPlan pl = ls::flow_plan(pairs, max_blocks, max_selected);
  f.chunks = pl.chunks;
  f.chunk_tiles = pl.chunk_tiles;
  f.splits = pl.splits;
  f.split = pl.split;
  f.n_refresh = (up.n_tiles + ls::kFlowWaves - 1) / ls::kFlowWaves;
  return f;
}

// Host-side validation of ls_sparse_decode_step's arguments (workspace aside).
ls_status check_step(const void* q, int32_t q_dtype, int32_t num_q_heads, const void* summaries,
                     const void* k_pool, const void* v_pool, const ls_pool& pool,
                     const ls_batch& batch, const ls_select_params* p, const int32_t* selected,
                     const int32_t* selected_count, float sm_scale, const void* out,
                     int32_t out_dtype, const int32_t* new_page_ids, int32_t n_new_pages) {
  if (!p) return fail(LS_ERR_INVALID, "params must be non-null");
  if (p->struct_size != (int32_t)sizeof(ls_select_params))
    return fail(LS_ERR_INVALID, "params.struct_size %d != %d", p->struct_size,
                (int)sizeof(ls_select_params));
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if ((st = check_gqa_pool(pool, "kv pool")) != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (out_dtype != LS_DTYPE_BF16 && out_dtype != LS_DTYPE_FP32)
    return fail(LS_ERR_UNSUPPORTED, "out_dtype %d (supported: bf16, fp32)", out_dtype);
  if (num_q_heads < 1 || num_q_heads % pool.num_heads != 0)
    return fail(LS_ERR_INVALID, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                pool.num_heads);
  if (!group_ok(num_q_heads / pool.num_heads))
    return fail(LS_ERR_UNSUPPORTED, "GQA group size %d (supported: 1, 2, 4, 8)",
                num_q_heads / pool.num_heads);
  if (p->group_agg != LS_AGG_MAX && p->group_agg != LS_AGG_MEAN)
    return fail(LS_ERR_INVALID, "group_agg %d", p->group_agg);
  if (p->score_mode != LS_SCORE_MEAN && p->score_mode != LS_SCORE_BOUNDS)
    return fail(LS_ERR_INVALID, "score_mode %d", p->score_mode);
  if (p->score_mode == LS_SCORE_BOUNDS && num_q_heads / pool.num_heads != 4)
    return fail(LS_ERR_UNSUPPORTED, "bounds scoring needs GQA group 4");
  if (p->score_mode == LS_SCORE_BOUNDS && batch.batch_size > 0 && !bounds_ok(pool, batch))
    return fail(LS_ERR_UNSUPPORTED,
                "bounds scoring needs max_blocks <= 8192 and num_pages < 2^26");
  if (p->n_sink < 0 || p->n_recent < 0) return fail(LS_ERR_INVALID, "n_sink/n_recent < 0");
  if (p->topk < -1) return fail(LS_ERR_INVALID, "topk %d (>= 0, or -1 for keep_ratio)", p->topk);
  if (p->topk == -1 && !(p->keep_ratio >= 0.0f && p->keep_ratio <= 1.0f))
    return fail(LS_ERR_INVALID, "keep_ratio must be in [0, 1]");
  if (!std::isfinite(sm_scale)) return fail(LS_ERR_INVALID, "sm_scale must be finite");
  if (n_new_pages < 0) return fail(LS_ERR_INVALID, "n_new_pages < 0");
  if (n_new_pages > 0 && !new_page_ids)
    return fail(LS_ERR_INVALID, "new_page_ids must be non-null when n_new_pages > 0");
  if (n_new_pages > 0 && p->n_recent < 1)
    return fail(LS_ERR_INVALID,
                "refreshing summaries in the step needs n_recent >= 1 (a page that just filled "
                "must not be scored in the same call)");
  if (batch.batch_size == 0) return ok();
  if (batch.max_blocks > 16384)
    return fail(LS_ERR_UNSUPPORTED, "max_blocks %d (supported: <= 16384)", batch.max_blocks);
  const int need = max_total_selected(*p, batch.max_blocks);
  if (p->max_selected < need)
    return fail(LS_ERR_INVALID, "max_selected %d < %d (largest possible selection)",
                p->max_selected, need);
  if (!q || !summaries || !k_pool || !v_pool || !selected || !selected_count || !out)
    return fail(LS_ERR_INVALID, "q, summaries, pools, selection and out must be non-null");
  if (!aligned16(q) || !aligned16(summaries) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(LS_ERR_INVALID, "q, summaries, k_pool and v_pool must be 16-byte aligned");
  return ok();
}

// The step over a validated workspace `w` laid out as `lay`.
ls_status run_step(const void* q, int32_t num_q_heads, void* summaries, const void* k_pool,
                   const void* v_pool, const ls_pool& pool, const ls_batch& batch,
                   const ls_select_params& p, int32_t* selected, int32_t* selected_count,
                   float sm_scale, void* out, int32_t out_dtype, float* lse_out,
                   const int32_t* new_page_ids, int32_t n_new_pages, char* w, const StepWs& lay,
                   hipStream_t stream) {
  float* scores = reinterpret_cast<float*>(w + lay.rows);
  float* partials = reinterpret_cast<float*>(w + lay.parts);
  const ls::ScoreArgs sa = score_args(q, num_q_heads, summaries, pool, batch, p, scores);
  if (const ls_status d = debug_check(sa.b, stream)) return d;
  const ls::TopkArgs ta = topk_args(sa, p, scores, selected, selected_count);
  const ls::AttnArgs aa = attn_args(q, num_q_heads, k_pool, v_pool, pool, batch, selected,
                                    selected_count, p.max_selected,
                                    ls_attn_num_splits(p.max_selected), sm_scale, partials, out,
                                    out_dtype, lse_out);
  const ls::SummaryUpdate up{static_cast<const uint16_t*>(k_pool), new_page_ids,
                             n_new_pages * pool.num_heads, summaries};
  const Route rt = route(pool, batch, num_q_heads);
  if (rt == kRouteItem) {
    ls::ScoreArgs si = sa;
    si.scores = nullptr;
    return hip_status(ls::launch_step_item(si, ta, aa, up, stream), "decode-step kernel launch");
  }
  if (rt == kRouteFlow) {
    const ls::FlowArgs f = flow_args(sa, ta, aa, up, batch.batch_size * pool.num_heads,
                                     batch.max_blocks, p.max_selected, w, lay.rows, lay.ents,
                                     lay.parts, nullptr);
    return hip_status(ls::launch_flow(f, ls::kFlowStep, stream), "decode-step kernel launch");
  }
  if (rt == kRoutePlan) {
    // the selection calls, then the attention call, as ls_score_select and
    // ls_sparse_attn_decode run them (same kernels, same bits; the ranker
    // also writes the selection's walk entries, which the attention reads
    // instead of the selection and the page table)
    const ls::PlanArgs pa = plan_args(sa, ta, aa, up, batch.batch_size * pool.num_heads,
                                      batch.max_blocks, w, lay.rows, lay.parts, nullptr, lay.ents);
    hipError_t e = ls::launch_plan_select(pa, stream);
    if (e == hipSuccess) e = ls::launch_plan_attend(pa, stream);
    return hip_status(e, "decode-step kernel launches");
  }
  // longer requests: the split kernels of the two calls back to back
  hipError_t e = hipSuccess;
  if (n_new_pages > 0) {
    const ls::SummaryArgs su{k_pool, nullptr, pool, new_page_ids, n_new_pages, summaries,
                             LS_DTYPE_BF16};
    e = ls::launch_summaries(su, stream);
    if (e != hipSuccess) return hip_status(e, "summary kernel launch");
  }
  e = ls::launch_score(sa, stream);
  if (e == hipSuccess) e = ls::launch_topk(ta, stream);
  if (e == hipSuccess) e = ls::launch_attn(aa, stream);
  // leave the workspace zero
  if (e == hipSuccess) e = ls::launch_zero(w + lay.rows, lay.total - lay.rows, stream);
  return hip_status(e, "decode-step kernel launches");
}

// ---- no-allocation step: a fixed device array instead of a caller workspace

// Bytes of the array; ls_sparse_decode_step_noalloc rejects shapes whose
// step workspace is larger.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kNoAllocMaxDevices = 64;

// One copy per GPU, held by the loaded library until the process ends. In
// host code the name is only a stand-in: the device address comes from
// hipGetSymbolAddress (scratch_ptr), and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// The calling thread's current device's copy of the array (looked up once
// per device, with that device current).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* ls_last_error(void) { return g_err; }

const char* ls_version(void) { return "libls 0.7.0 abi 6 gfx950"; }

int32_t ls_attn_num_splits(int32_t max_selected) {
  if (max_selected < 1) return 1;
  return (max_selected + ls::kAttnBlocksPerSplit - 1) / ls::kAttnBlocksPerSplit;
}

ls_status ls_build_block_summaries(const void* keys, const float* key_scales, ls_pool key_pool,
                                   const int32_t* page_ids, int32_t n_pages, void* summaries,
                                   int32_t summary_dtype, hipStream_t stream) {
  if (n_pages < 0) return fail(LS_ERR_INVALID, "n_pages < 0");
  if (key_pool.num_pages < 1 || key_pool.num_heads < 1)
    return fail(LS_ERR_INVALID, "key_pool: num_pages and num_heads must be >= 1");
  if (!pow2(key_pool.page_size) || key_pool.page_size < 16 || key_pool.page_size > 64)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.page_size %d (supported: 16, 32, 64)",
                key_pool.page_size);
  if (key_pool.head_dim != 64 && key_pool.head_dim != 128)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.head_dim %d (supported: 64, 128)", key_pool.head_dim);
  if (summary_dtype != LS_DTYPE_BF16 && summary_dtype != LS_DTYPE_FP32)
    return fail(LS_ERR_UNSUPPORTED, "summary_dtype %d (supported: bf16, fp32)", summary_dtype);
  if (key_pool.dtype == LS_DTYPE_BF16) {
    if (key_scales) return fail(LS_ERR_INVALID, "key_scales must be NULL for bf16 keys");
  } else if (key_pool.dtype == LS_DTYPE_FP8_E4M3FN) {
    if (!key_scales) return fail(LS_ERR_INVALID, "fp8 keys need key_scales");
    if (key_pool.num_heads != 1)
      return fail(LS_ERR_UNSUPPORTED, "fp8 key pools must have num_heads == 1");
  } else {
    return fail(LS_ERR_UNSUPPORTED, "key_pool.dtype %d (supported: bf16, fp8_e4m3fn)",
                key_pool.dtype);
  }
  if (n_pages == 0) return ok();
  if (!keys || !page_ids || !summaries)
    return fail(LS_ERR_INVALID, "keys, page_ids and summaries must be non-null");
  if (!aligned16(keys) || !aligned16(summaries))
    return fail(LS_ERR_INVALID, "keys and summaries must be 16-byte aligned");
  ls::SummaryArgs a{keys, key_scales, key_pool, page_ids, n_pages, summaries, summary_dtype};
  return hip_status(ls::launch_summaries(a, stream), "ls_build_block_summaries launch");
}

ls_status ls_build_block_bounds(const void* keys, ls_pool key_pool, const int32_t* page_ids,
                                int32_t n_pages, void* bounds, hipStream_t stream) {
  if (n_pages < 0) return fail(LS_ERR_INVALID, "n_pages < 0");
  if (key_pool.num_pages < 1 || key_pool.num_heads < 1)
    return fail(LS_ERR_INVALID, "key_pool: num_pages and num_heads must be >= 1");
  if (!pow2(key_pool.page_size) || key_pool.page_size < 16 || key_pool.page_size > 64)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.page_size %d (supported: 16, 32, 64)",
                key_pool.page_size);
  if (key_pool.head_dim != 64 && key_pool.head_dim != 128)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.head_dim %d (supported: 64, 128)", key_pool.head_dim);
  if (key_pool.dtype != LS_DTYPE_BF16)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.dtype %d (supported: bf16)", key_pool.dtype);
  if (n_pages == 0) return ok();
  if (!keys || !page_ids || !bounds)
    return fail(LS_ERR_INVALID, "keys, page_ids and bounds must be non-null");
  if (!aligned16(keys) || !aligned16(bounds))
    return fail(LS_ERR_INVALID, "keys and bounds must be 16-byte aligned");
  ls::SummaryArgs a{keys, nullptr, key_pool, page_ids, n_pages, bounds, LS_DTYPE_BF16};
  return hip_status(ls::launch_bounds(a, stream), "ls_build_block_bounds launch");
}

size_t ls_score_select_workspace_size(int32_t batch_size, int32_t num_kv_heads,
                                      int32_t max_blocks) {
  if (batch_size <= 0 || num_kv_heads <= 0 || max_blocks <= 0) return 0;
  return select_ws(batch_size, num_kv_heads, max_blocks).total;
}

ls_status ls_score_select(const void* q, int32_t q_dtype, int32_t num_q_heads,
                          const void* summaries, ls_pool pool, ls_batch batch,
                          const ls_select_params* p, int32_t* selected, int32_t* selected_count,
                          float* scores_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!p) return fail(LS_ERR_INVALID, "params must be non-null");
  if (p->struct_size != (int32_t)sizeof(ls_select_params))
    return fail(LS_ERR_INVALID, "params.struct_size %d != %d", p->struct_size,
                (int)sizeof(ls_select_params));
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if ((st = check_gqa_pool(pool, "summary pool")) != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (num_q_heads < 1 || num_q_heads % pool.num_heads != 0)
    return fail(LS_ERR_INVALID, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                pool.num_heads);
  if (!group_ok(num_q_heads / pool.num_heads))
    return fail(LS_ERR_UNSUPPORTED, "GQA group size %d (supported: 1, 2, 4, 8)",
                num_q_heads / pool.num_heads);
  if (p->group_agg != LS_AGG_MAX && p->group_agg != LS_AGG_MEAN)
    return fail(LS_ERR_INVALID, "group_agg %d", p->group_agg);
  if (p->score_mode != LS_SCORE_MEAN && p->score_mode != LS_SCORE_BOUNDS)
    return fail(LS_ERR_INVALID, "score_mode %d", p->score_mode);
  if (p->score_mode == LS_SCORE_BOUNDS && num_q_heads / pool.num_heads != 4)
    return fail(LS_ERR_UNSUPPORTED, "bounds scoring needs GQA group 4");
  if (p->score_mode == LS_SCORE_BOUNDS && batch.batch_size > 0 && !bounds_ok(pool, batch))
    return fail(LS_ERR_UNSUPPORTED,
                "bounds scoring needs max_blocks <= 8192 and num_pages < 2^26");
  if (p->n_sink < 0 || p->n_recent < 0) return fail(LS_ERR_INVALID, "n_sink/n_recent < 0");
  if (p->topk < -1) return fail(LS_ERR_INVALID, "topk %d (>= 0, or -1 for keep_ratio)", p->topk);
  if (p->topk == -1 && !(p->keep_ratio >= 0.0f && p->keep_ratio <= 1.0f))
    return fail(LS_ERR_INVALID, "keep_ratio must be in [0, 1]");
  if (batch.batch_size > 0 && batch.max_blocks > 16384)
    return fail(LS_ERR_UNSUPPORTED, "max_blocks %d (supported: <= 16384)", batch.max_blocks);
  if (batch.batch_size == 0) return ok();
  const int need = max_total_selected(*p, batch.max_blocks);
  if (p->max_selected < need)
    return fail(LS_ERR_INVALID, "max_selected %d < %d (largest possible selection)",
                p->max_selected, need);
  if (!q || !summaries || !selected || !selected_count)
    return fail(LS_ERR_INVALID, "q, summaries, selected and selected_count must be non-null");
  if (!aligned16(q) || !aligned16(summaries))
    return fail(LS_ERR_INVALID, "q and summaries must be 16-byte aligned");
  const SelectWs lay = select_ws(batch.batch_size, pool.num_heads, batch.max_blocks);
  if (!workspace || workspace_bytes < lay.total)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  char* w = static_cast<char*>(workspace);
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(w + lay.rows);
  const ls::ScoreArgs sa = score_args(q, num_q_heads, summaries, pool, batch, *p, scores);
  if (const ls_status d = debug_check(sa.b, stream)) return d;
  const ls::TopkArgs ta = topk_args(sa, *p, scores, selected, selected_count);
  const Route rt = route(pool, batch, num_q_heads);
  if (rt == kRouteItem) {
    ls::ScoreArgs si = sa;
    si.scores = scores_out;   // scores stay in LDS unless the caller asked for them
    return hip_status(ls::launch_select_item(si, ta, stream), "selection kernel launch");
  }
  if (rt == kRouteFlow) {
    const ls::FlowArgs f = flow_args(sa, ta, ls::AttnArgs{}, ls::SummaryUpdate{},
                                     batch.batch_size * pool.num_heads, batch.max_blocks,
                                     p->max_selected, w, lay.rows, 0, 0, scores_out);
    return hip_status(ls::launch_flow(f, ls::kFlowSelect, stream), "selection kernel launch");
  }
  if (rt == kRoutePlan) {
    const ls::PlanArgs pa = plan_args(sa, ta, ls::AttnArgs{}, ls::SummaryUpdate{},
                                      batch.batch_size * pool.num_heads, batch.max_blocks, w,
                                      lay.rows, 0, scores_out);
    return hip_status(ls::launch_plan_select(pa, stream), "selection kernel launches");
  }
  hipError_t e = ls::launch_score(sa, stream);
  if (e != hipSuccess) return hip_status(e, "score kernel launch");
  e = ls::launch_topk(ta, stream);
  if (e == hipSuccess && !scores_out) e = ls::launch_zero(w + lay.rows, lay.total - lay.rows, stream);
  return hip_status(e, "top-k kernel launch");
}

size_t ls_sparse_attn_decode_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_selected,
                                            int32_t max_blocks) {
  if (batch_size <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return attn_ws(batch_size, num_q_heads, head_dim, max_selected, max_blocks).total;
}

ls_status ls_sparse_attn_decode(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                const void* k_pool, const void* v_pool, ls_pool pool,
                                ls_batch batch, const int32_t* selected,
                                const int32_t* selected_count, int32_t max_selected,
                                float sm_scale, void* out, int32_t out_dtype, float* lse_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if ((st = check_gqa_pool(pool, "kv pool")) != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (out_dtype != LS_DTYPE_BF16 && out_dtype != LS_DTYPE_FP32)
    return fail(LS_ERR_UNSUPPORTED, "out_dtype %d (supported: bf16, fp32)", out_dtype);
  if (num_q_heads < 1 || num_q_heads % pool.num_heads != 0)
    return fail(LS_ERR_INVALID, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                pool.num_heads);
  if (!group_ok(num_q_heads / pool.num_heads))
    return fail(LS_ERR_UNSUPPORTED, "GQA group size %d (supported: 1, 2, 4, 8)",
                num_q_heads / pool.num_heads);
  if ((selected == nullptr) != (selected_count == nullptr))
    return fail(LS_ERR_INVALID, "selected and selected_count must both be set or both NULL");
  if (selected && max_selected < 1) return fail(LS_ERR_INVALID, "max_selected must be >= 1");
  if (!std::isfinite(sm_scale)) return fail(LS_ERR_INVALID, "sm_scale must be finite");
  if (batch.batch_size == 0) return ok();
  if (!q || !k_pool || !v_pool || !out)
    return fail(LS_ERR_INVALID, "q, k_pool, v_pool and out must be non-null");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(LS_ERR_INVALID, "q, k_pool and v_pool must be 16-byte aligned");
  const int cap = selected ? max_selected : batch.max_blocks;
  const AttnWs lay = attn_ws(batch.batch_size, num_q_heads, pool.head_dim,
                             selected ? max_selected : 0, batch.max_blocks);
  if (!workspace || workspace_bytes < lay.total)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  char* w = static_cast<char*>(workspace);
  float* partials = reinterpret_cast<float*>(w + lay.parts);
  const ls::AttnArgs aa = attn_args(q, num_q_heads, k_pool, v_pool, pool, batch, selected,
                                    selected_count, max_selected, ls_attn_num_splits(cap),
                                    sm_scale, partials, out, out_dtype, lse_out);
  if (const ls_status d = debug_check(aa.b, stream)) return d;
  // a selection: split over several workgroups per pair, merged by the last
  // one to finish; the dense path (every block) of few pairs is split-K over
  // runs of up to 512 blocks, merged by a second kernel
  const Route rt = route(pool, batch, num_q_heads);
  if (selected && rt == kRouteItem)
    return hip_status(ls::launch_attn_item(aa, stream), "attention kernel launch");
  if (selected && rt == kRouteFlow) {
    const ls::FlowArgs f = flow_args(ls::ScoreArgs{}, ls::TopkArgs{}, aa, ls::SummaryUpdate{},
                                     batch.batch_size * pool.num_heads, batch.max_blocks,
                                     max_selected, w, 0, 0, lay.parts, nullptr);
    return hip_status(ls::launch_flow(f, ls::kFlowAttend, stream), "attention kernel launch");
  }
  // every block (dense) of at least kItemMinPairs pairs: the planned
  // kernel too (ranges balanced over the pairs, whatever their lengths)
  const int pairs = batch.batch_size * pool.num_heads;
  const bool plan_dense = !selected && pairs >= ls::kItemMinPairs &&
                          ls::plan_ok(num_q_heads / pool.num_heads, pool.head_dim,
                                      batch.max_blocks, pool.num_pages, pairs);
  if (rt == kRoutePlan || plan_dense) {   // a selection, or every block (dense)
    const ls::PlanArgs pa = plan_args(ls::ScoreArgs{}, ls::TopkArgs{}, aa, ls::SummaryUpdate{},
                                      pairs, batch.max_blocks, w, 0, lay.parts, nullptr);
    return hip_status(ls::launch_plan_attend(pa, stream), "attention kernel launch");
  }
  const bool chunked = !selected && num_q_heads == 4 * pool.num_heads && pool.num_pages < (1 << 26);
  hipError_t e = chunked ? ls::launch_attn_chunked(aa, stream) : ls::launch_attn(aa, stream);
  // leave the workspace zero
  if (e == hipSuccess) e = ls::launch_zero(w + lay.parts, lay.total - lay.parts, stream);
  return hip_status(e, "attention kernel launch");
}

size_t ls_sparse_decode_step_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks, int32_t max_selected) {
  if (batch_size <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks <= 0 || max_selected <= 0)
    return 0;
  return step_ws(batch_size, num_q_heads, num_kv_heads, head_dim, max_blocks, max_selected).total;
}

ls_status ls_sparse_decode_step(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                void* summaries, const void* k_pool, const void* v_pool,
                                ls_pool pool, ls_batch batch, const ls_select_params* p,
                                int32_t* selected, int32_t* selected_count, float sm_scale,
                                void* out, int32_t out_dtype, float* lse_out,
                                const int32_t* new_page_ids, int32_t n_new_pages, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  const ls_status st = check_step(q, q_dtype, num_q_heads, summaries, k_pool, v_pool, pool, batch,
                                  p, selected, selected_count, sm_scale, out, out_dtype,
                                  new_page_ids, n_new_pages);
  if (st != LS_OK || batch.batch_size == 0) return st;
  const StepWs lay = step_ws(batch.batch_size, num_q_heads, pool.num_heads, pool.head_dim,
                             batch.max_blocks, p->max_selected);
  if (!workspace || workspace_bytes < lay.total)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  return run_step(q, num_q_heads, summaries, k_pool, v_pool, pool, batch, *p, selected,
                  selected_count, sm_scale, out, out_dtype, lse_out, new_page_ids, n_new_pages,
                  static_cast<char*>(workspace), lay, stream);
}

size_t ls_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int32_t ls_stream_read_sink_words(void) { return ls::kStreamReadWorkgroups; }

ls_status ls_check_batch(ls_batch batch, int32_t page_size, int32_t num_pages, int32_t* report,
                         hipStream_t stream) {
  if (!report || (uintptr_t)report % 4)
    return fail(LS_ERR_INVALID, "report must be a non-null, 4-byte aligned device pointer");
  if (page_size < 1 || num_pages < 1)
    return fail(LS_ERR_INVALID, "page_size and num_pages must be >= 1");
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  ls::BatchArgs b;
  b.batch = batch.batch_size;
  b.max_blocks = batch.max_blocks;
  b.indptr = batch.page_indptr;
  b.indices = batch.page_indices;
  b.seq_lens = batch.seq_lens;
  b.num_pages = num_pages;
  b.page_size = page_size;
  return hip_status(ls::launch_batch_check(b, report, false, stream), "batch check launch");
}

void ls_debug_enable(int32_t on) { g_debug.store(on ? 1 : 0); }

int32_t ls_debug_enabled(void) { return debug_on() ? 1 : 0; }

ls_status ls_debug_report(int32_t* host_report) {
  if (!host_report) return fail(LS_ERR_INVALID, "host_report must be non-null");
  int32_t* words = nullptr;
  hipError_t e = debug_words_ptr(&words);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(host_report, words, 4 * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(words, 0, 4 * sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return hip_status(e, "debug report");
}

ls_status ls_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(LS_ERR_INVALID, "src and sink must be non-null");
  if (!aligned16(src) || bytes % 16)
    return fail(LS_ERR_INVALID, "src must be 16-byte aligned and bytes a multiple of 16");
  return hip_status(ls::launch_stream_read(src, bytes, sink, ls::kStreamReadWorkgroups, stream),
                    "stream read launch");
}

ls_status ls_sparse_decode_step_noalloc(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                        void* summaries, const void* k_pool, const void* v_pool,
                                        ls_pool pool, ls_batch batch, const ls_select_params* p,
                                        int32_t* selected, int32_t* selected_count,
                                        float sm_scale, void* out, int32_t out_dtype,
                                        float* lse_out, const int32_t* new_page_ids,
                                        int32_t n_new_pages, hipStream_t stream) {
  const ls_status st = check_step(q, q_dtype, num_q_heads, summaries, k_pool, v_pool, pool, batch,
                                  p, selected, selected_count, sm_scale, out, out_dtype,
                                  new_page_ids, n_new_pages);
  if (st != LS_OK || batch.batch_size == 0) return st;
  const StepWs lay = step_ws(batch.batch_size, num_q_heads, pool.num_heads, pool.head_dim,
                             batch.max_blocks, p->max_selected);
  if (lay.total > kNoAllocScratchBytes)
    return fail(LS_ERR_UNSUPPORTED,
                "ls_sparse_decode_step_noalloc: this shape needs %zu bytes of scratch, more than "
                "the library's fixed %zu (use ls_sparse_decode_step with a workspace)",
                lay.total, kNoAllocScratchBytes);
  void* w = nullptr;
  hipError_t e = scratch_ptr(&w);
  if (e != hipSuccess) return hip_status(e, "scratch address lookup");
  // the step expects a zero workspace; the array keeps the last call's
  // contents (zero after every call that completed), so clear what this
  // call uses first (a fill kernel: capturable in a graph)
  e = ls::launch_zero(w, lay.total, stream);
  if (e != hipSuccess) return hip_status(e, "scratch clear launch");
  return run_step(q, num_q_heads, summaries, k_pool, v_pool, pool, batch, *p, selected,
                  selected_count, sm_scale, out, out_dtype, lse_out, new_page_ids, n_new_pages,
                  static_cast<char*>(w), lay, stream);
}

// ------------------------------------------------------ learned indexer ----

int32_t ls_indexer_score_stride(int32_t granularity, int32_t max_units) {
  if (max_units <= 0) return 0;
  if (granularity == LS_SEL_BLOCKS) return max_units;
  return (max_units + ls::kIdxMarkUnits - 1) / ls::kIdxMarkUnits * ls::kIdxMarkUnits;
}

size_t ls_indexer_select_workspace_size(int32_t batch_size, int32_t granularity,
                                        int32_t max_units) {
  if (batch_size <= 0 || max_units <= 0) return 0;
  const size_t B = (size_t)batch_size;
  const size_t U = (size_t)ls_indexer_score_stride(granularity, max_units);
  size_t ws = align_up(B * U * sizeof(float));   // scores
  if (granularity == LS_SEL_TOKENS) {
    ws += align_up(B * ls::kIdxCoarse * sizeof(uint32_t));              // bucket histograms
    ws += align_up(B * 4 * sizeof(uint32_t));                         // counters, remap
    ws += align_up(B * (U / ls::kIdxMinWgUnits) * sizeof(float2));    // score ranges
    ws += align_up(B * U * sizeof(uint2));                            // threshold-bucket units
    ws += align_up(B * (U / 32) * sizeof(uint32_t));                  // bitmap
  }
  return ws;
}

// Scoring tiles (16 units each) per workgroup: up to 128, fewer while that
// leaves fewer than LS_IDX_MIN_WGS workgroups (the scoring loop is bound by
// issue and latency, so the chip needs several waves per SIMD).
#ifndef LS_IDX_MIN_WGS
#define LS_IDX_MIN_WGS 512
#endif
static int indexer_tiles_per_wg(size_t B, int U) {
  int tiles = 128;
  while (tiles > 4 && (long long)B * ((U + 16 * tiles - 1) / (16 * tiles)) < LS_IDX_MIN_WGS)
    tiles /= 2;
  return tiles;
}

// The token top-k's part of the workspace (after the scores), in the order
// ls_indexer_select_workspace_size counts it.
static void token_topk_layout(ls::IndexerArgs& a, char* w, size_t B, int U) {
  a.hist = reinterpret_cast<uint32_t*>(w);
  w += align_up(B * ls::kIdxCoarse * sizeof(uint32_t));
  a.ctl = reinterpret_cast<uint32_t*>(w);
  w += align_up(B * 4 * sizeof(uint32_t));
  a.range = reinterpret_cast<float2*>(w);
  w += align_up(B * (U / ls::kIdxMinWgUnits) * sizeof(float2));
  a.cand = reinterpret_cast<uint2*>(w);
  w += align_up(B * U * sizeof(uint2));
  a.bitmap = reinterpret_cast<uint32_t*>(w);
}

ls_status ls_indexer_select(const void* q, int32_t q_dtype, int32_t num_heads,
                            const float* head_weights, const void* keys, const float* key_scales,
                            ls_pool key_pool, ls_batch batch, const int32_t* cand_blocks,
                            const int32_t* cand_counts, int32_t cand_cap,
                            const ls_indexer_params* p, int32_t* selected,
                            int32_t* selected_count, float* scores_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!p) return fail(LS_ERR_INVALID, "params must be non-null");
  if (p->struct_size != (int32_t)sizeof(ls_indexer_params))
    return fail(LS_ERR_INVALID, "params.struct_size %d != %d", p->struct_size,
                (int)sizeof(ls_indexer_params));
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  const bool tokens = p->granularity == LS_SEL_TOKENS;
  if (!tokens && p->granularity != LS_SEL_BLOCKS)
    return fail(LS_ERR_INVALID, "granularity %d (LS_SEL_TOKENS or LS_SEL_BLOCKS)", p->granularity);
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (num_heads != 16 && num_heads != 32 && num_heads != 64)
    return fail(LS_ERR_UNSUPPORTED, "num_heads %d (supported: 16, 32, 64)", num_heads);
  if (key_pool.num_pages < 1) return fail(LS_ERR_INVALID, "key_pool.num_pages must be >= 1");
  if (key_pool.num_heads != 1)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.num_heads %d (supported: 1)", key_pool.num_heads);
  if (key_pool.head_dim != 128)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.head_dim %d (supported: 128)", key_pool.head_dim);
  if (key_pool.page_size != 16 && key_pool.page_size != 32 && key_pool.page_size != 64)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.page_size %d (supported: 16, 32, 64)",
                key_pool.page_size);
  if (p->topk < 0) return fail(LS_ERR_INVALID, "topk %d must be >= 0", p->topk);
  if (p->n_sink < 0 || p->n_recent < 0) return fail(LS_ERR_INVALID, "n_sink/n_recent < 0");
  if (p->candidates != LS_CAND_BLOCKS && p->candidates != LS_CAND_TOKENS)
    return fail(LS_ERR_INVALID, "candidates %d (LS_CAND_BLOCKS or LS_CAND_TOKENS)",
                p->candidates);
  const bool tok_cands = p->candidates == LS_CAND_TOKENS;
  if (p->approx < 0 || p->approx > 1) return fail(LS_ERR_INVALID, "approx %d (0 or 1)", p->approx);
  if (p->approx && !tokens) return fail(LS_ERR_UNSUPPORTED, "approx is for LS_SEL_TOKENS");
  if (tok_cands && (!tokens || !cand_blocks))
    return fail(LS_ERR_INVALID, "LS_CAND_TOKENS needs LS_SEL_TOKENS and a candidate list");
  if (tok_cands && (long long)key_pool.num_pages * key_pool.page_size >= (1ll << 31))
    return fail(LS_ERR_UNSUPPORTED, "LS_CAND_TOKENS needs num_pages * page_size < 2^31");
  int max_units;
  if (tokens) {
    if (key_pool.dtype != LS_DTYPE_FP8_E4M3FN)
      return fail(LS_ERR_UNSUPPORTED, "token keys must be fp8_e4m3fn");
    if (p->n_sink || p->n_recent)
      return fail(LS_ERR_UNSUPPORTED, "forced units are supported for blocks only");
    if (cand_blocks) {
      if (!cand_counts || cand_cap < 1)
        return fail(LS_ERR_INVALID, "cand_blocks needs cand_counts and cand_cap >= 1");
      max_units = tok_cands ? cand_cap + key_pool.page_size : cand_cap * key_pool.page_size;
    } else {
      max_units = batch.max_blocks * key_pool.page_size;
    }
    if (batch.batch_size > 0 && (max_units < 1 || max_units > ls::kIdxMaxUnits))
      return fail(LS_ERR_UNSUPPORTED, "%d tokens per request (supported: <= %d)", max_units,
                  ls::kIdxMaxUnits);
    if (p->max_selected < p->topk)
      return fail(LS_ERR_INVALID, "max_selected %d < topk %d", p->max_selected, p->topk);
  } else {
    if (key_pool.dtype != LS_DTYPE_BF16)
      return fail(LS_ERR_UNSUPPORTED, "block summaries must be bf16");
    if (key_scales) return fail(LS_ERR_INVALID, "key_scales must be NULL for block summaries");
    if (cand_blocks) return fail(LS_ERR_UNSUPPORTED, "candidate lists are for tokens only");
    if (batch.batch_size > 0 && batch.max_blocks > 16384)
      return fail(LS_ERR_UNSUPPORTED, "max_blocks %d (supported: <= 16384)", batch.max_blocks);
    max_units = batch.max_blocks;
    const long long need = std::min<long long>(batch.max_blocks,
                                               (long long)p->topk + p->n_sink + p->n_recent + 1);
    if (p->max_selected < need)
      return fail(LS_ERR_INVALID, "max_selected %d < %lld (largest possible selection)",
                  p->max_selected, need);
  }
  if (batch.batch_size == 0) return ok();
  if (!q || !head_weights || !keys || !selected || !selected_count)
    return fail(LS_ERR_INVALID, "q, head_weights, keys, selected and selected_count must be non-null");
  if (!aligned16(q) || !aligned16(keys))
    return fail(LS_ERR_INVALID, "q and keys must be 16-byte aligned");
  const size_t ws = ls_indexer_select_workspace_size(batch.batch_size, p->granularity, max_units);
  if (!workspace || workspace_bytes < ws)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, ws);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);

  const size_t B = (size_t)batch.batch_size;
  const int U = ls_indexer_score_stride(p->granularity, max_units);
  char* w = static_cast<char*>(workspace);
  ls::IndexerArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.w = head_weights;
  a.keys = keys;
  a.scales = key_scales;
  a.b = batch_args(batch, key_pool);
  a.num_heads = num_heads;
  a.cand_blocks = cand_blocks;
  a.cand_counts = cand_counts;
  a.cand_cap = cand_cap;
  a.unit_kind = tok_cands ? ls::kUnitsTokenCands : ls::kUnitsDefault;
  a.approx = p->approx;
  a.max_units = U;
  a.n_sink = p->n_sink;
  a.n_recent = p->n_recent;
  a.scores = scores_out ? scores_out : reinterpret_cast<float*>(w);
  w += align_up(B * U * sizeof(float));
  a.topk = p->topk;
  a.max_selected = p->max_selected;
  a.selected = selected;
  a.selected_count = selected_count;
  a.tiles_per_wg = indexer_tiles_per_wg(B, U);
  if (const ls_status d = debug_check(a.b, stream)) return d;
  if (!tokens) {
    hipError_t e = ls::launch_indexer_score(a, ls::kIdxBlocks, stream);
    if (e != hipSuccess) return hip_status(e, "indexer score kernel launch");
    ls::TopkArgs ta{};
    ta.scores = a.scores;
    ta.b = a.b;
    ta.num_kv_heads = 1;
    ta.topk = p->topk;
    ta.keep_ratio = 0.0f;
    ta.n_sink = p->n_sink;
    ta.n_recent = p->n_recent;
    ta.max_selected = p->max_selected;
    ta.selected = selected;
    ta.selected_count = selected_count;
    return hip_status(ls::launch_topk(ta, stream), "top-k kernel launch");
  }
  token_topk_layout(a, w, B, U);
  return hip_status(ls::launch_indexer_token_select(a, stream), "indexer selection launches");
}

// ------------------------------------------------------------ sparse MLA ----

int32_t ls_mla_num_splits(int32_t max_tokens) {
  if (max_tokens < 1) return 1;
  return (max_tokens + ls::kMlaSplitTokens - 1) / ls::kMlaSplitTokens;
}

size_t ls_sparse_mla_decode_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                           int32_t max_tokens) {
  if (batch_size <= 0 || num_q_heads <= 0) return 0;
  const size_t rows = (size_t)batch_size * num_q_heads * ls_mla_num_splits(max_tokens);
  return align_up(rows * 2 * sizeof(float)) + align_up(rows * 512 * sizeof(float));
}

ls_status ls_sparse_mla_decode(const void* q, int32_t q_dtype, int32_t num_q_heads,
                               const void* latent, ls_pool pool, ls_batch batch,
                               const int32_t* selected, const int32_t* selected_count,
                               int32_t max_selected, float sm_scale, void* out,
                               int32_t out_dtype, float* lse_out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (out_dtype != LS_DTYPE_BF16 && out_dtype != LS_DTYPE_FP32)
    return fail(LS_ERR_UNSUPPORTED, "out_dtype %d (supported: bf16, fp32)", out_dtype);
  if (pool.num_pages < 1) return fail(LS_ERR_INVALID, "pool.num_pages must be >= 1");
  if (pool.num_heads != 1 || pool.head_dim != 576 || pool.dtype != LS_DTYPE_BF16)
    return fail(LS_ERR_UNSUPPORTED, "latent pool must be bf16 with num_heads 1 and head_dim 576");
  if (pool.page_size < 1 || pool.page_size > 1024)
    return fail(LS_ERR_UNSUPPORTED, "pool.page_size %d (supported: 1 .. 1024)", pool.page_size);
  if (num_q_heads < 32 || num_q_heads > 256 || num_q_heads % 32 != 0)
    return fail(LS_ERR_UNSUPPORTED, "num_q_heads %d (supported: multiples of 32 up to 256)",
                num_q_heads);
  if ((selected == nullptr) != (selected_count == nullptr))
    return fail(LS_ERR_INVALID, "selected and selected_count must both be set or both NULL");
  if (selected && max_selected < 1) return fail(LS_ERR_INVALID, "max_selected must be >= 1");
  if (!std::isfinite(sm_scale)) return fail(LS_ERR_INVALID, "sm_scale must be finite");
  if (batch.batch_size == 0) return ok();
  if (!q || !latent || !out) return fail(LS_ERR_INVALID, "q, latent and out must be non-null");
  if (!aligned16(q) || !aligned16(latent))
    return fail(LS_ERR_INVALID, "q and latent must be 16-byte aligned");
  const long long dense = (long long)batch.max_blocks * pool.page_size;
  if (!selected && dense > (1 << 24))
    return fail(LS_ERR_UNSUPPORTED, "dense MLA over %lld tokens (supported: <= 2^24)", dense);
  const int cap = selected ? max_selected : (int)dense;
  const size_t ws = ls_sparse_mla_decode_workspace_size(batch.batch_size, num_q_heads, cap);
  if (!workspace || workspace_bytes < ws)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, ws);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  ls::MlaArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.latent = static_cast<const uint16_t*>(latent);
  a.b = batch_args(batch, pool);
  a.num_q_heads = num_q_heads;
  a.selected = selected;
  a.selected_count = selected_count;
  a.max_selected = selected ? max_selected : 0;
  a.num_splits = ls_mla_num_splits(cap);
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.partials = static_cast<float*>(workspace);
  a.out = out;
  a.out_dtype = out_dtype;
  a.lse = lse_out;
  if (const ls_status d = debug_check(a.b, stream)) return d;
  return hip_status(ls::launch_mla(a, stream), "MLA kernel launches");
}


// ---------------------------------------------------- sink + window ----

namespace {

int window_positions(int32_t max_blocks, int32_t n_sink, int32_t window) {
  const long long p = ((long long)n_sink + 15) / 16 + ((long long)window + 15) / 16 + 1;
  return (int)std::min<long long>(p, (long long)max_blocks + 1);
}

}  // namespace

size_t ls_window_attn_decode_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_blocks, int32_t n_sink,
                                            int32_t window) {
  if (batch_size <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks <= 0 || n_sink < 0 ||
      window < 0)
    return 0;
  const size_t S = (size_t)ls_attn_num_splits(window_positions(max_blocks, n_sink, window));
  return align_up((size_t)batch_size * num_q_heads * S * (head_dim + 2) * sizeof(float));
}

ls_status ls_window_attn_decode(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                const void* k_pool, const void* v_pool, ls_pool pool,
                                ls_batch batch, int32_t n_sink, int32_t window, float sm_scale,
                                void* out, int32_t out_dtype, float* lse_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if ((st = check_gqa_pool(pool, "kv pool")) != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (out_dtype != LS_DTYPE_BF16 && out_dtype != LS_DTYPE_FP32)
    return fail(LS_ERR_UNSUPPORTED, "out_dtype %d (supported: bf16, fp32)", out_dtype);
  if (num_q_heads < 1 || num_q_heads % pool.num_heads != 0)
    return fail(LS_ERR_INVALID, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                pool.num_heads);
  if (num_q_heads / pool.num_heads != 4)
    return fail(LS_ERR_UNSUPPORTED, "GQA group size %d (supported: 4)",
                num_q_heads / pool.num_heads);
  if (n_sink < 0 || window < 0) return fail(LS_ERR_INVALID, "n_sink and window must be >= 0");
  if (pool.num_pages >= (1 << 22))
    return fail(LS_ERR_UNSUPPORTED, "num_pages %d (supported: < 2^22)", pool.num_pages);
  if (!std::isfinite(sm_scale)) return fail(LS_ERR_INVALID, "sm_scale must be finite");
  if (batch.batch_size == 0) return ok();
  if (!q || !k_pool || !v_pool || !out)
    return fail(LS_ERR_INVALID, "q, k_pool, v_pool and out must be non-null");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(LS_ERR_INVALID, "q, k_pool and v_pool must be 16-byte aligned");
  const int npos = window_positions(batch.max_blocks, n_sink, window);
  const size_t ws = ls_window_attn_decode_workspace_size(batch.batch_size, num_q_heads,
                                                         pool.head_dim, batch.max_blocks, n_sink,
                                                         window);
  if (!workspace || workspace_bytes < ws)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, ws);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  ls::AttnArgs aa = attn_args(q, num_q_heads, k_pool, v_pool, pool, batch, nullptr, nullptr, 0,
                              ls_attn_num_splits(npos), sm_scale,
                              static_cast<float*>(workspace), out, out_dtype, lse_out);
  aa.win_sink = n_sink;
  aa.win_len = window;
  if (const ls_status d = debug_check(aa.b, stream)) return d;
  return hip_status(ls::launch_attn_window(aa, npos, stream), "window attention launches");
}

// ------------------------------------------------------ SnapKV selection ----

namespace {

struct SnapLayout {
  size_t stats, rowstat, scores, keys, total;
};

SnapLayout snap_layout(int batch_size, int num_kv_heads, int max_len) {
  const size_t pairs = (size_t)batch_size * num_kv_heads;
  const size_t n_chunks = ((size_t)max_len + 255) / 256;
  const size_t cells = pairs * (size_t)max_len;
  SnapLayout l{};
  size_t o = 0;
  l.stats = o;   o += align_up(pairs * n_chunks * ls::kSnapMaxObs * 4 * 2 * sizeof(float));
  l.rowstat = o; o += align_up(pairs * ls::kSnapMaxObs * 4 * 2 * sizeof(float));
  l.scores = o;  o += align_up(cells * sizeof(float));
  l.keys = o;    o += align_up(cells * sizeof(float));
  l.total = o;
  return l;
}

}  // namespace

size_t ls_snapkv_select_workspace_size(int32_t batch_size, int32_t num_kv_heads,
                                       int32_t max_len) {
  if (batch_size <= 0 || num_kv_heads <= 0 || max_len <= 0 || max_len > ls::kSnapMaxLen) return 0;
  return snap_layout(batch_size, num_kv_heads, max_len).total;
}

ls_status ls_snapkv_select(const void* q_obs, int32_t q_dtype, int32_t num_q_heads,
                           int32_t n_obs, const void* k_pool, ls_pool pool, ls_batch batch,
                           int32_t max_len, float sm_scale, int32_t n_sink, int32_t budget,
                           int32_t* selected, int32_t* counts, float* scores_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if ((st = check_gqa_pool(pool, "kv pool")) != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (num_q_heads != 4 * pool.num_heads)
    return fail(LS_ERR_UNSUPPORTED, "GQA group size must be 4");
  if (n_obs < 1 || n_obs > ls::kSnapMaxObs)
    return fail(LS_ERR_UNSUPPORTED, "n_obs %d (supported: 1 .. %d)", n_obs, ls::kSnapMaxObs);
  if (max_len < 1 || max_len > ls::kSnapMaxLen)
    return fail(LS_ERR_UNSUPPORTED, "max_len %d (supported: 1 .. %d)", max_len, ls::kSnapMaxLen);
  if ((long long)max_len * batch.batch_size * pool.num_heads >= (1ll << 31))
    return fail(LS_ERR_UNSUPPORTED, "batch * kv heads * max_len must be < 2^31");
  if (n_sink < 0 || budget < 1) return fail(LS_ERR_INVALID, "n_sink >= 0 and budget >= 1");
  if (!std::isfinite(sm_scale)) return fail(LS_ERR_INVALID, "sm_scale must be finite");
  if (batch.batch_size == 0) return ok();
  if (!q_obs || !k_pool || !selected || !counts)
    return fail(LS_ERR_INVALID, "q_obs, k_pool, selected and counts must be non-null");
  if (!aligned16(q_obs) || !aligned16(k_pool))
    return fail(LS_ERR_INVALID, "q_obs and k_pool must be 16-byte aligned");
  const SnapLayout l = snap_layout(batch.batch_size, pool.num_heads, max_len);
  if (!workspace || workspace_bytes < l.total)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, l.total);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  char* w = static_cast<char*>(workspace);
  const size_t pairs = (size_t)batch.batch_size * pool.num_heads;
  ls::SnapArgs a{};
  a.q_obs = static_cast<const uint16_t*>(q_obs);
  a.n_obs = n_obs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool.num_heads;
  a.head_dim = pool.head_dim;
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.b = batch_args(batch, pool);
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.n_sink = n_sink;
  a.budget = budget;
  a.max_len = max_len;
  a.n_chunks = (max_len + 255) / 256;
  a.stats = reinterpret_cast<float*>(w + l.stats);
  a.rowstat = reinterpret_cast<float*>(w + l.rowstat);
  a.scores = scores_out ? scores_out : reinterpret_cast<float*>(w + l.scores);
  a.keys = reinterpret_cast<float*>(w + l.keys);
  a.selected = selected;
  a.counts = counts;
  if (const ls_status d = debug_check(a.b, stream)) return d;
  return hip_status(ls::launch_snapkv_select(a, stream), "SnapKV selection launches");
}

ls_status ls_snapkv_gather(const void* k_pool, const void* v_pool, ls_pool pool, ls_batch batch,
                           const int32_t* selected, const int32_t* counts, int32_t budget,
                           void* k_out, void* v_out, hipStream_t stream) {
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  if ((st = check_gqa_pool(pool, "kv pool")) != LS_OK) return st;
  if (budget < 1) return fail(LS_ERR_INVALID, "budget must be >= 1");
  if (batch.batch_size == 0) return ok();
  if (!k_pool || !v_pool || !selected || !counts || !k_out || !v_out)
    return fail(LS_ERR_INVALID, "pools, selection and outputs must be non-null");
  ls::SnapArgs a{};
  a.num_kv_heads = pool.num_heads;
  a.head_dim = pool.head_dim;
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.b = batch_args(batch, pool);
  a.budget = budget;
  a.selected = const_cast<int32_t*>(selected);
  a.counts = const_cast<int32_t*>(counts);
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  const int budget_pad = (budget + 15) / 16 * 16;
  if (const ls_status d = debug_check(a.b, stream)) return d;
  return hip_status(ls::launch_snapkv_gather(a, budget_pad, stream), "SnapKV gather launch");
}

// ------------------------------------------------------------------ PQ32 ----

namespace {

ls_status check_pq_pool(const ls_pool& key_pool) {
  if (key_pool.num_pages < 1) return fail(LS_ERR_INVALID, "key_pool.num_pages must be >= 1");
  if (key_pool.num_heads != 1 || key_pool.head_dim != 128)
    return fail(LS_ERR_UNSUPPORTED, "key_pool: num_heads 1 and head_dim 128 (got %d, %d)",
                key_pool.num_heads, key_pool.head_dim);
  if (key_pool.page_size != 16 && key_pool.page_size != 32 && key_pool.page_size != 64)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.page_size %d (supported: 16, 32, 64)",
                key_pool.page_size);
  if (key_pool.dtype != LS_DTYPE_FP8_E4M3FN)
    return fail(LS_ERR_UNSUPPORTED, "key_pool.dtype must be fp8_e4m3fn");
  return LS_OK;
}

}  // namespace

ls_status ls_pq_encode(const void* keys, const float* key_scales, ls_pool key_pool,
                       const int32_t* page_ids, int32_t n_pages, const void* codebooks,
                       uint8_t* codes, hipStream_t stream) {
  ls_status st = check_pq_pool(key_pool);
  if (st != LS_OK) return st;
  if (n_pages < 0) return fail(LS_ERR_INVALID, "n_pages < 0");
  if (n_pages == 0) return ok();
  if (!keys || !page_ids || !codebooks || !codes)
    return fail(LS_ERR_INVALID, "keys, page_ids, codebooks and codes must be non-null");
  if ((uintptr_t)keys % 4 || (uintptr_t)codebooks % 16)
    return fail(LS_ERR_INVALID, "keys must be 4-byte and codebooks 16-byte aligned");
  ls::PqArgs a{static_cast<const uint8_t*>(keys), key_scales, key_pool.num_pages,
               key_pool.page_size, page_ids, n_pages,
               const_cast<uint16_t*>(static_cast<const uint16_t*>(codebooks)), codes, nullptr,
               nullptr};
  return hip_status(ls::launch_pq_encode(a, stream), "PQ encode launch");
}

size_t ls_pq_train_workspace_size(void) {
  return align_up((size_t)ls::kPqSub * ls::kPqCent * ls::kPqDim * sizeof(unsigned long long)) +
         align_up((size_t)ls::kPqSub * ls::kPqCent * sizeof(uint32_t));
}

ls_status ls_pq_train(const void* keys, const float* key_scales, ls_pool key_pool,
                      const int32_t* page_ids, int32_t n_pages, const int32_t* init_tokens,
                      int32_t iters, void* codebooks, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  ls_status st = check_pq_pool(key_pool);
  if (st != LS_OK) return st;
  if (n_pages < 1) return fail(LS_ERR_INVALID, "n_pages must be >= 1");
  if (iters < 0 || iters > 1000) return fail(LS_ERR_INVALID, "iters %d (0 .. 1000)", iters);
  if ((long long)n_pages * key_pool.page_size > (1ll << 31) - 1)
    return fail(LS_ERR_UNSUPPORTED, "more than 2^31 - 1 training tokens");
  if (!keys || !page_ids || !init_tokens || !codebooks)
    return fail(LS_ERR_INVALID, "keys, page_ids, init_tokens and codebooks must be non-null");
  if ((uintptr_t)keys % 4 || (uintptr_t)codebooks % 16)
    return fail(LS_ERR_INVALID, "keys must be 4-byte and codebooks 16-byte aligned");
  if (!workspace || workspace_bytes < ls_pq_train_workspace_size())
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                ls_pq_train_workspace_size());
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  char* w = static_cast<char*>(workspace);
  auto* sums = reinterpret_cast<unsigned long long*>(w);
  auto* counts = reinterpret_cast<uint32_t*>(
      w + align_up((size_t)ls::kPqSub * ls::kPqCent * ls::kPqDim * sizeof(unsigned long long)));
  ls::PqArgs a{static_cast<const uint8_t*>(keys), key_scales, key_pool.num_pages,
               key_pool.page_size, page_ids, n_pages, static_cast<uint16_t*>(codebooks), nullptr,
               sums, counts};
  return hip_status(ls::launch_pq_train(a, init_tokens, iters, stream), "PQ training launches");
}

ls_status ls_pq_select(const void* q, int32_t q_dtype, int32_t num_heads,
                       const float* head_weights, const uint8_t* codes, const void* codebooks,
                       ls_pool key_pool, ls_batch batch, int32_t n_candidates,
                       int32_t* candidates, int32_t* candidate_counts, float* scores_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ls_status st = check_batch(batch);
  if (st != LS_OK) return st;
  st = check_pq_pool(key_pool);
  if (st != LS_OK) return st;
  if (q_dtype != LS_DTYPE_BF16) return fail(LS_ERR_UNSUPPORTED, "q_dtype must be bf16");
  if (num_heads != 16 && num_heads != 32 && num_heads != 64)
    return fail(LS_ERR_UNSUPPORTED, "num_heads %d (supported: 16, 32, 64)", num_heads);
  if (n_candidates < 0) return fail(LS_ERR_INVALID, "n_candidates %d must be >= 0", n_candidates);
  const long long mu = (long long)batch.max_blocks * key_pool.page_size;
  if (batch.batch_size > 0 && (mu < 1 || mu > ls::kIdxMaxUnits))
    return fail(LS_ERR_UNSUPPORTED, "%lld tokens per request (supported: <= %d)", mu,
                ls::kIdxMaxUnits);
  if (batch.batch_size == 0) return ok();
  if (!q || !head_weights || !codes || !codebooks || !candidates || !candidate_counts)
    return fail(LS_ERR_INVALID,
                "q, head_weights, codes, codebooks, candidates and counts must be non-null");
  if (!aligned16(q) || (uintptr_t)codebooks % 16 || (uintptr_t)codes % 8)
    return fail(LS_ERR_INVALID, "q and codebooks must be 16-byte, codes 8-byte aligned");
  const int max_units = (int)mu;
  const size_t ws = ls_indexer_select_workspace_size(batch.batch_size, LS_SEL_TOKENS, max_units);
  if (!workspace || workspace_bytes < ws)
    return fail(LS_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, ws);
  if ((uintptr_t)workspace % kAlign)
    return fail(LS_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  const size_t B = (size_t)batch.batch_size;
  const int U = ls_indexer_score_stride(LS_SEL_TOKENS, max_units);
  char* w = static_cast<char*>(workspace);
  ls::IndexerArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.w = head_weights;
  a.keys = codes;
  a.codebooks = static_cast<const uint16_t*>(codebooks);
  a.b = batch_args(batch, key_pool);
  a.num_heads = num_heads;
  a.unit_kind = ls::kUnitsComplete;
  a.max_units = U;
  a.scores = scores_out ? scores_out : reinterpret_cast<float*>(w);
  w += align_up(B * U * sizeof(float));
  a.topk = n_candidates;
  a.max_selected = n_candidates;
  a.selected = candidates;
  a.selected_count = candidate_counts;
  a.tiles_per_wg = indexer_tiles_per_wg(B, U);
  token_topk_layout(a, w, B, U);
  if (const ls_status d = debug_check(a.b, stream)) return d;
  return hip_status(ls::launch_pq_select(a, stream), "PQ selection launches");
}

ls_status ls_pq_filter_misses(const int32_t* candidates, const int32_t* candidate_counts,
                              int32_t cap, const float* scores, int32_t score_stride,
                              const uint32_t* resident, int32_t resident_words,
                              int32_t batch_size, int32_t topk, int32_t* kept,
                              int32_t* kept_counts, int32_t* misses_kept, hipStream_t stream) {
  if (batch_size < 0) return fail(LS_ERR_INVALID, "batch_size %d must be >= 0", batch_size);
  if (cap < 1 || cap > ls::kPqFilterMaxCand)
    return fail(LS_ERR_UNSUPPORTED, "cap %d (supported: 1 .. %d)", cap, ls::kPqFilterMaxCand);
  if (score_stride < 1) return fail(LS_ERR_INVALID, "score_stride %d must be >= 1", score_stride);
  if (resident_words < 0) return fail(LS_ERR_INVALID, "resident_words %d must be >= 0", resident_words);
  if (topk < 1) return fail(LS_ERR_INVALID, "topk %d must be >= 1", topk);
  if (batch_size == 0) return ok();
  if (!candidates || !candidate_counts || !scores || !kept || !kept_counts)
    return fail(LS_ERR_INVALID, "candidates, counts, scores, kept and kept_counts must be non-null");
  if (resident_words > 0 && !resident)
    return fail(LS_ERR_INVALID, "resident must be non-null when resident_words > 0");
  ls::PqFilterArgs a{};
  a.candidates = candidates;
  a.counts = candidate_counts;
  a.cap = cap;
  a.scores = scores;
  a.score_stride = score_stride;
  a.resident = resident;
  a.resident_words = resident_words;
  a.topk = topk;
  a.kept = kept;
  a.kept_counts = kept_counts;
  a.misses_kept = misses_kept;
  return hip_status(ls::launch_pq_filter(a, batch_size, stream), "PQ miss filter launch");
}

}  // extern "C"

// Internal launch interface between the C ABI layer (ls_api.hip) and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include "../../include/ls.h"
#include "ls_device.h"

namespace ls {

struct SummaryArgs {
  const void* keys;
  const float* key_scales;
  ls_pool pool;
  const int32_t* page_ids;
  int32_t n_pages;
  void* out;
  int32_t out_dtype;
};

// Per-request geometry shared by scoring, selection and attention.
struct BatchArgs {
  int32_t batch;
  int32_t max_blocks;
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* seq_lens;
  int32_t num_pages;
  int32_t page_size;
};

struct ScoreArgs {
  const uint16_t* q;          // [B][Hq][D] bf16
  const uint16_t* summaries;  // [num_pages][Hkv][D] bf16
  BatchArgs b;
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t group_agg;
  int32_t n_sink, n_recent;
  float* scores;              // [B][Hkv][max_blocks]
  int32_t bounds;             // 1: summaries are Quest bounds [num_pages][Hkv][2][D]
};

struct TopkArgs {
  const float* scores;        // [B][Hkv][max_blocks]
  BatchArgs b;
  int32_t num_kv_heads;
  int32_t topk;
  float keep_ratio;
  int32_t n_sink, n_recent;
  int32_t max_selected;
  int32_t* selected;          // [B][Hkv][max_selected]
  int32_t* selected_count;    // [B][Hkv]
};

struct AttnArgs {
  const uint16_t* q;          // [B][Hq][D]
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  BatchArgs b;
  int32_t num_q_heads, num_kv_heads, head_dim;
  const int32_t* selected;    // nullptr => dense (every block)
  const int32_t* selected_count;
  int32_t max_selected;       // row stride of `selected`
  int32_t num_splits;
  float sm_scale_log2;        // sm_scale * log2(e)
  float* partials;            // [B][Hq][S][D+2]
  void* out;
  int32_t out_dtype;
  float* lse;
  int32_t win_sink, win_len;  // window attention: sinks [0, win_sink) + the last win_len tokens
};

hipError_t launch_summaries(const SummaryArgs& a, hipStream_t st);
// Quest bounds (bf16 keys): out = [num_pages][num_heads][2][D] bf16.
hipError_t launch_bounds(const SummaryArgs& a, hipStream_t st);

// Pages whose bf16 summaries a decode step refreshes alongside its work
// (pages that just filled; n_tiles = pages * kv heads, 0 = none).
struct SummaryUpdate {
  const uint16_t* keys;     // K pool [num_pages][Hkv][P][D]
  const int32_t* pages;
  int32_t n_tiles;
  void* out;                // summary pool [num_pages][Hkv][D] bf16
};
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
// The combine kernel alone: merges a.num_splits partials per query head.
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st);

// Per-(request, kv head) kernels (one 1024-thread workgroup per pair), used
// when there are at least kItemMinPairs pairs: the selection and the
// attention of a pair then fit one workgroup each, with no cross-workgroup
// merge. ScoreArgs.scores may be null for these (scores stay in LDS).
constexpr int kItemMinPairs = 64;
bool item_path(int batch, int hkv, int head_dim, int group, int max_blocks, int num_pages);
// Requests of more than kPairMinBlocks blocks, in batches of at most
// kPairMaxPairs pairs, take two workgroups per pair (scoring split in half,
// attention positions interleaved, softmax states merged by the second to
// finish): the one-workgroup step does not fit in LDS there, and the grid
// still covers the chip. The attention workspace then holds the pairs'
// exchange areas (2 * 4 * D + 16 floats each, rounded) followed by their
// arrival counters.
constexpr int kPairMaxPairs = 256;
constexpr int kPairMinBlocks = 4096;
bool pair_path(int batch, int hkv, int max_blocks);
inline size_t pair_workspace_bytes(int pairs, int head_dim) {
  const size_t f = (size_t)pairs * (2 * 4 * head_dim + 16) * sizeof(float);
  return (f + 255) / 256 * 256 + (size_t)pairs * sizeof(uint32_t);
}
inline uint32_t* pair_arrivals(float* partials, int pairs, int head_dim) {
  const size_t f = (size_t)pairs * (2 * 4 * head_dim + 16) * sizeof(float);
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(partials) + (f + 255) / 256 * 256);
}
hipError_t launch_select_item(const ScoreArgs& sa, const TopkArgs& ta, hipStream_t st);
hipError_t launch_attn_item(const AttnArgs& a, hipStream_t st);
// Split-K with the per-pair attention body: each workgroup attends a run of
// up to kChunkMaxBlocks consecutive positions of a pair's selection (of its
// block list on the dense path), then the combine kernel merges the runs.
// Needs num_pages < 2^26; a.num_splits on entry is the capacity of the
// partials (splits of kAttnBlocksPerSplit), which the chunking never exceeds.
constexpr int kChunkMaxBlocks = 512;
hipError_t launch_attn_chunked(const AttnArgs& a, hipStream_t st);
// Sink + recent window: tokens [0, min(win_sink, L)) and [max(that, L -
// win_len), L) of every request, in place, split over runs of positions like
// the dense path (max_pos: positions per pair at most).
hipError_t launch_attn_window(const AttnArgs& a, int max_pos, hipStream_t st);
hipError_t launch_step_item(const ScoreArgs& sa, const TopkArgs& ta, const AttnArgs& aa,
                            const SummaryUpdate& up, hipStream_t st);

// Learned-indexer selection (k_indexer.hip): scoring of tokens (fp8 keys) or
// blocks (bf16 block-mean keys) and the token top-k.
constexpr int kIdxBins = 4096;          // buckets of the remapped score
constexpr int kIdxCoarse = 256;         // first digit: bucket >> 4 (the histogram's bins)
constexpr int kIdxMarkUnits = 4096;     // units per mark workgroup (score row strides are multiples)
constexpr int kIdxMinWgUnits = 64;      // units per scoring workgroup at least (score-range slots)
constexpr int kIdxMaxUnits = 262144;    // units per request (token mode)

enum { kIdxTokens = 0, kIdxBlocks = 1 };
// Units of a request in token mode: every cached token, or the tokens of the
// candidate blocks (kUnitsDefault); the candidate tokens, then the tokens of
// the partial last page (kUnitsTokenCands); the tokens of the complete pages
// (kUnitsComplete, PQ coarse scoring).
enum { kUnitsDefault = 0, kUnitsTokenCands = 1, kUnitsComplete = 2 };

struct IndexerArgs {
  const uint16_t* q;           // [B][H][128] bf16
  const float* w;              // [B][H]
  const void* keys;            // tokens: fp8 [num_pages][P][128]; blocks: bf16 [num_pages][128]
  const float* scales;         // tokens: [num_pages][P] or null (1); blocks: unused
  BatchArgs b;
  int32_t num_heads;
  const int32_t* cand_blocks;  // tokens, optional: [B][cand_cap] ascending block ids
                               // (token ids with kUnitsTokenCands)
  int32_t unit_kind;           // kUnits*
  int32_t approx;              // tokens: 1 = fill from the boundary bucket in unit order
  const uint16_t* codebooks;   // PQ coarse scoring: [32][256][4] bf16 (keys = codes)
  const int32_t* cand_counts;  // [B]
  int32_t cand_cap;
  int32_t max_units;           // row stride of scores (units per request, max)
  int32_t tiles_per_wg;        // multiple of 4, <= 128
  int32_t n_sink, n_recent;    // blocks mode: forced blocks (not scored)
  float* scores;               // [B][max_units]
  float2* range;               // tokens: [B][max_units / kIdxMinWgUnits] (min, max) of the
                               // valid scores of each scoring workgroup
  uint32_t* hist;              // tokens: [B][kIdxCoarse] first-digit histogram
  int32_t topk;
  int32_t max_selected;
  uint32_t* ctl;               // tokens: [B][4] (candidates, arrivals, remap min, remap scale)
  uint2* cand;                 // tokens: [B][max_units] (key, unit) of the threshold bucket
  uint32_t* bitmap;            // tokens: [B][max_units / 32]
  int32_t* selected;           // tokens: [B][max_selected]
  int32_t* selected_count;     // tokens: [B]
};

hipError_t launch_indexer_score(const IndexerArgs& a, int mode, hipStream_t st);
// the token top-k after the scoring (which leaves every workgroup's score
// range and clears the request's histogram and counters): the histogram of
// the remapped scores, then mark + finish
hipError_t launch_indexer_hist(const IndexerArgs& a, hipStream_t st);
hipError_t launch_indexer_mark(const IndexerArgs& a, hipStream_t st);
// PQ32 coarse selection (k_pq.hip): coarse scores of the complete pages'
// tokens from their codes, histogram, mark + finish
hipError_t launch_pq_select(const IndexerArgs& a, hipStream_t st);

// One-time SnapKV-style selection and gather (k_snapkv.hip).
constexpr int kSnapMaxObs = 64;        // observation queries
constexpr int kSnapMaxLen = 131072;    // cache positions per request
struct SnapArgs {
  const uint16_t* q_obs;     // [B][n_obs][Hq][D] bf16
  int32_t n_obs, num_q_heads, num_kv_heads, head_dim;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  BatchArgs b;
  float sm_scale_log2;
  int32_t n_sink, budget, max_len, n_chunks;
  float* stats;              // [pairs][n_chunks][4 kSnapMaxObs][2]
  float* rowstat;            // [pairs][4 kSnapMaxObs][2]
  float* scores;             // [pairs][max_len]
  float* keys;               // [pairs][max_len] the candidates' averaged scores
  int32_t* selected;         // [pairs][budget]
  int32_t* counts;           // [pairs]
  uint16_t* k_out;           // gather: [pairs][budget_pad][D]
  uint16_t* v_out;
};
hipError_t launch_snapkv_select(const SnapArgs& a, hipStream_t st);
hipError_t launch_snapkv_gather(const SnapArgs& a, int budget_pad, hipStream_t st);

// PQ32 codes and codebooks (k_pq.hip).
constexpr int kPqSub = 32, kPqCent = 256, kPqDim = 4, kPqFixedBits = 24;
struct PqArgs {
  const uint8_t* keys;          // fp8 e4m3fn [num_pages][P][128]
  const float* scales;          // [num_pages][P], or null (1)
  int32_t num_pages, page_size;
  const int32_t* page_ids;      // the listed pages; token i = slot i % P of page_ids[i / P]
  int32_t n_pages;
  uint16_t* codebooks;          // [32][256][4] bf16
  uint8_t* codes;               // encode: [num_pages][P][32]
  unsigned long long* sums;     // training: [32][256][4] fixed-point sums
  uint32_t* counts;             // training: [32][256]
};
hipError_t launch_pq_encode(const PqArgs& a, hipStream_t st);
hipError_t launch_pq_train(const PqArgs& a, const int32_t* init_tokens, int iters,
                           hipStream_t st);
// score, histogram, mark + finish (three launches)
hipError_t launch_indexer_token_select(const IndexerArgs& a, hipStream_t st);

// Miss filter over PQ candidates (k_pq.hip): one workgroup per request.
constexpr int kPqFilterMaxCand = 4096;   // candidates per request
struct PqFilterArgs {
  const int32_t* candidates;   // [B][cap] token ids, ascending
  const int32_t* counts;       // [B]
  int32_t cap;
  const float* scores;         // [B][score_stride] approximate score at token t
  int32_t score_stride;
  const uint32_t* resident;    // [B][resident_words] bit t: token t's key is resident
  int32_t resident_words;
  int32_t topk;
  int32_t* kept;               // [B][cap] (may be candidates itself)
  int32_t* kept_counts;        // [B]
  int32_t* misses_kept;        // [B] or null
};
hipError_t launch_pq_filter(const PqFilterArgs& a, int batch, hipStream_t st);

// Sparse MLA attention (k_mla.hip): one workgroup per (request, 16 query
// heads, kMlaSplitTokens selected tokens), then a log-sum-exp combine.
constexpr int kMlaSplitTokens = 256;

struct MlaArgs {
  const uint16_t* q;          // [B][H][576] bf16
  const uint16_t* latent;     // [num_pages][P][576] bf16
  BatchArgs b;
  int32_t num_q_heads;
  const int32_t* selected;    // [B][max_selected] token ids, or null (every cached token)
  const int32_t* selected_count;
  int32_t max_selected;
  int32_t num_splits;
  float sm_scale_log2;
  float* partials;            // (m, l) [B][H][S][2], then o [B][H][S][512] (fp32 or bf16)
  void* out;                  // [B][H][512]
  int32_t out_dtype;
  float* lse;
};

hipError_t launch_mla(const MlaArgs& a, hipStream_t st);

// Measurement reference (k_probe.hip): one streaming read of `bytes` bytes
// (2048 workgroups of four waves measured best on MI355X).
constexpr int kStreamReadWorkgroups = 2048;
// Debug check of a batch's device data (ls_check_batch, and LS_DEBUG): one
// workgroup; report = the caller's 4 words (overwritten) or the library's
// debug words (accumulated).
hipError_t launch_batch_check(const BatchArgs& b, int32_t* report, bool accumulate,
                              hipStream_t stream);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t st);

// Blocks per attention split (one register-resident chunk per workgroup).
constexpr int kAttnBlocksPerSplit = 8;

// Request geometry on the device: blocks, complete blocks, and the candidate
// range [c0, c1) = complete blocks that are neither sink nor recent. The
// block count is clamped to the pages the request owns and to max_blocks, so
// a request that breaks the page-table contract cannot make a kernel read
// outside its page list.
struct ReqGeom {
  int L, nb, nc, c0, c1, page_base;
};

__device__ __forceinline__ ReqGeom req_geom(const BatchArgs& b, int r, int n_sink, int n_recent) {
  ReqGeom g;
  int L = b.seq_lens[r];
  L = L < 0 ? 0 : L;
  const int p0 = b.indptr[r], p1 = b.indptr[r + 1];
  int npg = p1 - p0;
  npg = npg < 0 ? 0 : npg;
  int nb = (L + b.page_size - 1) / b.page_size;
  const int cap = npg < b.max_blocks ? npg : b.max_blocks;
  if (nb > cap) {
    nb = cap;
    L = nb * b.page_size;
  }
  g.L = L;
  g.nb = nb;
  g.nc = L / b.page_size;
  const int s = n_sink < nb ? n_sink : nb;
  int rec = nb - n_recent;
  rec = rec < 0 ? 0 : rec;
  g.c0 = s;
  g.c1 = g.nc < rec ? g.nc : rec;
  if (g.c1 < g.c0) g.c1 = g.c0;
  g.page_base = p0;
  return g;
}

}  // namespace ls

/*
 * ls.h -- C ABI of libls, a gfx950 (MI355X) library for the decode-step
 * query-aware sparse-attention hot path:
 *
 *   1. ls_build_block_summaries: the mean key of every full page, per KV head
 *      (Vortex post, "Writing an algorithm: vFlow": the block-top-k cache
 *      step stores the mean of the keys over the in-block axis; summaries are
 *      built once, when a block fills up -- "Why Long Generations Are
 *      Expensive").
 *   2. ls_score_select: score each block summary against the current query,
 *      aggregate over the query heads of a GQA group, and keep the top-k
 *      blocks plus forced sink / recent blocks (Vortex, block top-k equation
 *      and Fig. 1; the vFlow listing's GeMM -> head reduction -> topK).
 *   3. ls_sparse_attn_decode: exact softmax attention of every query head over
 *      the tokens of the selected blocks of a paged KV cache, split over the
 *      selected blocks and merged by log-sum-exp (Vortex block top-k
 *      equation; the merge of attention over disjoint token sets by
 *      log-sum-exp in "Where Activation Sparsity and KV-Cache Sparsity Cross
 *      in LLM Decoding", App. A).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer (hipMalloc'ed or equivalent) unless the
 *   comment says "host". The caller owns every buffer. The library allocates
 *   no device memory, keeps no pointer after a call returns (beyond the work
 *   it enqueued), never synchronises the stream and never reads device data
 *   back to the host, so every call can be captured in a HIP graph.
 * - Every call only ENQUEUES kernels on `stream` (0 = the null stream).
 * - Host-side validation runs before any launch. On failure nothing is
 *   enqueued, the call returns a non-zero ls_status, and ls_last_error()
 *   returns a message (thread-local, valid until the next call on the same
 *   thread). A launch error is reported as LS_ERR_HIP with the HIP message.
 *   The library never aborts and never throws across this ABI.
 * - Device-side contract (not checkable on the host without a readback):
 *   page ids < pool.num_pages; page_indptr non-decreasing; every request r
 *   has at least ceil(seq_lens[r] / page_size) pages; seq_lens[r] >= 0 and
 *   ceil(seq_lens[r]/page_size) <= batch.max_blocks; selection entries are
 *   ascending valid block indices. The kernels guard every such index before
 *   using it as an address (no out-of-bounds access), but results for a
 *   request that violates the contract are unspecified.
 * - Paged pool layout ("HND"): element (page, head, slot, d) of a K or V pool
 *   is at ((page * num_heads + head) * page_size + slot) * head_dim + d, so
 *   one (page, head) tile is contiguous. Logical block j of request r (tokens
 *   j*page_size ... j*page_size + page_size - 1) lives in physical page
 *   page_indices[page_indptr[r] + j] (the paged layout of the Vortex post,
 *   "Why New Ideas Are Hard to Deploy", Fig. 2). Block = page.
 * - Summary pool layout: [num_pages][num_heads][head_dim], indexed by
 *   PHYSICAL page id, so pages shared between requests share a summary
 *   (Vortex, "Running it: vTensor": cache entries live in pages of the KV
 *   allocator).
 * - bf16 is IEEE binary32's upper half; fp8 is OCP e4m3fn.
 * - Workspaces of ls_score_select, ls_sparse_attn_decode and
 *   ls_sparse_decode_step: device memory the caller zero-fills before its
 *   first use (e.g. hipMemset once at allocation). Every call leaves it zero
 *   again, so it can be reused by later calls of any of the three (not by
 *   calls running concurrently). Inside a call, workgroups hand data to
 *   each other through it (block scores, walk entries of the selection,
 *   partial softmax states): a word is zero until written, the reader polls
 *   it and writes zero back. Word 0 is an error word: non-zero after a call
 *   means a workgroup gave up waiting for a hand-off (never expected; that
 *   call's results are then unspecified).
 */
#ifndef LS_H_
#define LS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LS_ABI_VERSION 6

typedef enum ls_status {
  LS_OK = 0,
  LS_ERR_INVALID = 1,      /* bad argument: null pointer, negative size, mismatch */
  LS_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype / shape combination) */
  LS_ERR_WORKSPACE = 3,    /* workspace_bytes smaller than the size query returns */
  LS_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} ls_status;

typedef enum ls_dtype {
  LS_DTYPE_BF16 = 1,
  LS_DTYPE_FP32 = 2,
  LS_DTYPE_FP8_E4M3FN = 3
} ls_dtype;

/* GQA aggregation of the per-head block scores of one KV group. */
enum { LS_AGG_MAX = 0, LS_AGG_MEAN = 1 };

/* Block scores (ls_select_params.score_mode). */
enum { LS_SCORE_MEAN = 0, LS_SCORE_BOUNDS = 1 };

/* Geometry of a paged pool (K, V or summaries). */
typedef struct ls_pool {
  int32_t num_pages;   /* physical pages in the pool                     */
  int32_t num_heads;   /* KV heads per page                              */
  int32_t page_size;   /* tokens per page (= block size)                 */
  int32_t head_dim;    /* elements per token per head                    */
  int32_t dtype;       /* ls_dtype of the pool's elements                */
} ls_pool;

/* A ragged batch of requests over a paged pool (CSR page table, the
 * "index-pointer array" + page list of the Vortex post's vTensor).
 * Device data that breaks the contract is not undefined behaviour: every
 * kernel clamps a request's length to its page list and to max_blocks
 * pages (the tokens past them are not cached), takes a negative length as
 * 0, and reads nothing at a page id outside [0, num_pages) (such a block
 * scores 0 and its tokens are not attended), so no access leaves the
 * buffers whose sizes the call states. */
typedef struct ls_batch {
  int32_t batch_size;            /* host: number of requests (0 is allowed)  */
  int32_t max_blocks;            /* host: >= ceil(seq_lens[r]/page_size), all r */
  const int32_t* page_indptr;    /* [batch_size + 1]                         */
  const int32_t* page_indices;   /* [page_indptr[batch_size]] physical pages */
  const int32_t* seq_lens;       /* [batch_size] cached tokens, current one included */
} ls_batch;

/* Selection parameters (passed by host pointer). */
typedef struct ls_select_params {
  int32_t struct_size;   /* = sizeof(ls_select_params)                        */
  int32_t group_agg;     /* LS_AGG_MAX or LS_AGG_MEAN                         */
  int32_t topk;          /* blocks chosen by score, forced ones not counted;  */
                         /* -1 => per request from keep_ratio (below)         */
  float keep_ratio;      /* used when topk == -1: a request with nb blocks    */
                         /* keeps max(|F|, ceil(keep_ratio*nb)) blocks in all,*/
                         /* forced blocks F included                          */
  int32_t n_sink;        /* forced: blocks 0 .. n_sink-1                      */
  int32_t n_recent;      /* forced: the last n_recent blocks                  */
  int32_t max_selected;  /* row capacity of `selected` (see ls_score_select)  */
  int32_t score_mode;    /* LS_SCORE_MEAN: summaries are block-mean keys      */
                         /*   [num_pages][num_heads][head_dim];               */
                         /* LS_SCORE_BOUNDS: summaries are Quest bounds from  */
                         /*   ls_build_block_bounds,                          */
                         /*   [num_pages][num_heads][2][head_dim]             */
} ls_select_params;

/* ------------------------------------------------------------------------ */
/* 1. Block summaries                                                        */
/* ------------------------------------------------------------------------ */
/*
 * summaries[p][h][d] = round( (1/page_size) * sum_s keys[p][h][s][d] )
 * for every physical page p listed in page_ids[0 .. n_pages-1] and every
 * head h < key_pool.num_heads. The sum over the page's tokens is accumulated
 * in float64 (exact whenever, within one column, the largest and smallest
 * non-zero |key| are less than 2^41 apart), page_size is a power of two so the
 * division is exact, and the mean is rounded ONCE, to nearest-even, to
 * summary_dtype.
 *
 * keys:        key pool, layout HND (see above), dtype key_pool.dtype;
 *              16-byte aligned.
 * key_scales:  NULL for bf16 keys. For LS_DTYPE_FP8_E4M3FN keys: per-token
 *              dequantisation scale, fp32 [num_pages][page_size] (the summand
 *              is key_scales[p][s] * keys[p][h][s][d]); key_pool.num_heads
 *              must then be 1.
 * key_pool:    page_size in {16, 32, 64}; head_dim in {64, 128}; dtype bf16 or fp8.
 * page_ids:    [n_pages] physical page ids to (re)summarise (complete pages).
 * n_pages:     >= 0; 0 enqueues nothing.
 * summaries:   [key_pool.num_pages][key_pool.num_heads][head_dim] of
 *              summary_dtype (LS_DTYPE_BF16 or LS_DTYPE_FP32), 16-byte
 *              aligned; only the rows of the listed pages are written.
 * Errors: LS_ERR_INVALID for a null or misaligned pointer, LS_ERR_UNSUPPORTED
 *   for a geometry or dtype outside the sets above.
 */
ls_status ls_build_block_summaries(const void* keys, const float* key_scales,
                                   ls_pool key_pool, const int32_t* page_ids,
                                   int32_t n_pages, void* summaries,
                                   int32_t summary_dtype, hipStream_t stream);

/*
 * Quest bounds (Vortex post, "Writing an algorithm: vFlow", the Quest
 * listing: its cache step keeps the element-wise maximum and minimum key of
 * each block):
 *   bounds[p][h][0][d] = max_s keys[p][h][s][d],
 *   bounds[p][h][1][d] = min_s keys[p][h][s][d]
 * for every listed page p and head h. Exact (a copy of bf16 values). Keys
 * are taken to be finite.
 *
 * keys:     bf16 key pool, layout HND, 16-byte aligned; key_pool.dtype =
 *           LS_DTYPE_BF16, page_size in {16, 32, 64}, head_dim in {64, 128}.
 * page_ids: [n_pages] physical page ids (complete pages); n_pages >= 0.
 * bounds:   bf16 [key_pool.num_pages][key_pool.num_heads][2][head_dim],
 *           16-byte aligned; only the rows of the listed pages are written.
 */
ls_status ls_build_block_bounds(const void* keys, ls_pool key_pool, const int32_t* page_ids,
                                int32_t n_pages, void* bounds, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 2. Scoring and selection                                                  */
/* ------------------------------------------------------------------------ */
/*
 * For every request r and KV head g (G = num_q_heads / num_kv_heads query
 * heads per group, query head h belongs to group h / G):
 *   nb = ceil(L/P) blocks, nc = floor(L/P) complete blocks (L = seq_lens[r]),
 *   forced F = {0 .. min(n_sink,nb)-1} U {max(0,nb-n_recent) .. nb-1}
 *              U {nb-1 if the last block is partial},
 *   candidates C = {j < nc} \ F,
 *   score s_j = agg_{h in group g} u_h(j), unscaled, fp32 accumulation of
 *              exact bf16 products, with
 *     LS_SCORE_MEAN:   u_h(j) = sum_d q[r][h][d] * summaries[page(r,j)][g][d]
 *                      (Vortex post, block top-k equation),
 *     LS_SCORE_BOUNDS: u_h(j) = sum_d max(q[r][h][d] * bounds[page][g][0][d],
 *                                         q[r][h][d] * bounds[page][g][1][d])
 *                      (Vortex post, the Quest listing: an upper bound of
 *                      q . k over the block's keys),
 *   k_r = topk, or from keep_ratio when topk == -1,
 *   top = the first min(k_r, |C|) candidates ordered by (s_j descending,
 *         j ascending) -- ties go to the LOWEST block index,
 *   selected[r][g][0 .. cnt-1] = F U top in ASCENDING order, cnt = |F U top|,
 *   remaining entries up to max_selected set to -1, selected_count[r][g] = cnt.
 * The result is deterministic (bitwise identical run to run).
 *
 * q:              [batch][num_q_heads][head_dim], q_dtype = LS_DTYPE_BF16.
 * summaries:      summary pool [num_pages][num_kv_heads][head_dim]; its
 *                 geometry is `pool` (pool.num_heads = num_kv_heads,
 *                 pool.page_size = block size, pool.dtype = LS_DTYPE_BF16).
 * batch:          page table of the requests (block = page).
 * p:              host pointer; p->max_selected must be >= the largest
 *                 possible cnt, i.e. >= min(max_blocks, k + n_sink + n_recent + 1)
 *                 (k_max from keep_ratio when topk == -1).
 * selected:       [batch][num_kv_heads][p->max_selected] int32 (output).
 * selected_count: [batch][num_kv_heads] int32 (output).
 * scores_out:     NULL, or [batch][num_kv_heads][max_blocks] fp32 receiving
 *                 s_j for candidate blocks (other entries unspecified).
 * workspace:      device scratch of at least ls_score_select_workspace_size()
 *                 bytes, 256-byte aligned, always required (also with
 *                 scores_out); zero-filled before its first use (every
 *                 call leaves it zero, see "Workspaces" below).
 * Execution: one workgroup per (request, kv head) pair scores and ranks it
 *                 in LDS when there are at least 64 pairs of at most 4096
 *                 blocks. At least 64 pairs of longer requests (or fewer
 *                 pairs of more than 8192 blocks) take two launches planned
 *                 from the lengths: the candidate summary tiles of all pairs
 *                 are cut into equal ranges, one per scoring workgroup, then
 *                 one workgroup per pair ranks it. Fewer pairs of at most
 *                 8192 blocks take one launch in which workgroups score
 *                 chunks of 64-128 blocks and the pair's last chunk ranks it.
 *                 Other shapes take a scoring kernel and a top-k kernel.
 * Supported: head_dim in {64, 128}; num_q_heads / num_kv_heads in
 *            {1, 2, 4, 8}; page_size 16; max_blocks <= 16384
 *            (LS_SCORE_BOUNDS: group 4, max_blocks <= 8192, num_pages < 2^26).
 *            Groups other than 4 run on the operator-per-kernel route
 *            (scoring, top-k, split attention and combine as separate
 *            launches); group 4 takes the matrix-core routes above.
 */
size_t ls_score_select_workspace_size(int32_t batch_size, int32_t num_kv_heads,
                                      int32_t max_blocks);

ls_status ls_score_select(const void* q, int32_t q_dtype, int32_t num_q_heads,
                          const void* summaries, ls_pool pool, ls_batch batch,
                          const ls_select_params* p, int32_t* selected,
                          int32_t* selected_count, float* scores_out,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 3. Sparse attention over the selected blocks                              */
/* ------------------------------------------------------------------------ */
/*
 * For every request r and query head h (group g = h / G):
 *   T = tokens t < L of the blocks selected[r][g][0 .. cnt-1],
 *   z_t = sm_scale * sum_d q[r][h][d] * K[t][d],
 *   out[r][h][:] = sum_t e^{z_t - M} V[t][:] / sum_t e^{z_t - M}, M = max z,
 *   lse_out[r][h] = M + ln sum_t e^{z_t - M}
 * with fp32 logits, softmax and accumulation; partial softmax states over
 * disjoint token sets are merged by log-sum-exp in a fixed order
 * (deterministic). Batches of at least 64 pairs whose requests exceed 4096
 * blocks, and the dense path of at least 64 pairs, are planned from the
 * counts: the positions of all pairs (selected blocks, or every block) are
 * cut into equal ranges, one per workgroup of a fixed grid; a pair inside
 * one range is written by its workgroup, a pair cut by range ends is merged
 * in range order by the last of its workgroups to finish. Other selections
 * (requests of at most 8192 blocks) are split over workgroups of at most 16
 * selected blocks per (request, kv head) pair, merged the same way by the
 * pair's last workgroup. The dense path of fewer pairs splits each pair
 * into runs of up to 512 blocks whose states a second kernel merges
 * (split-K); longer requests take the split-K kernels of 8 blocks per split.
 * An empty T gives out = 0 and lse = -inf. The output is rounded once
 * (nearest-even) to out_dtype.
 * For a selection written by ls_score_select the entries past the count are
 * -1; other callers may leave them undefined (they are never read as blocks).
 *
 * q:              [batch][num_q_heads][head_dim] bf16.
 * k_pool, v_pool: K and V pools, layout HND, geometry `pool` (bf16).
 * selected:       [batch][num_kv_heads][max_selected] ascending block
 *                 indices (as written by ls_score_select), with counts in
 *                 selected_count[batch][num_kv_heads]. selected == NULL and
 *                 selected_count == NULL select EVERY block of each request
 *                 (the dense "k = all" path; max_selected is then ignored).
 * sm_scale:       logit scale, e.g. 1/sqrt(head_dim).
 * out:            [batch][num_q_heads][head_dim] of out_dtype (bf16 or fp32).
 * lse_out:        NULL or [batch][num_q_heads] fp32.
 * workspace:      >= ls_sparse_attn_decode_workspace_size() bytes, 256-byte
 *                 aligned (split partial results); zero-filled before its
 *                 first use (every call leaves it zero).
 * Supported: head_dim in {64, 128}; num_q_heads / num_kv_heads in
 *            {1, 2, 4, 8} (other than 4: the split kernels, selection or
 *            dense); page_size 16.
 */
size_t ls_sparse_attn_decode_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_selected,
                                            int32_t max_blocks);

ls_status ls_sparse_attn_decode(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                const void* k_pool, const void* v_pool, ls_pool pool,
                                ls_batch batch, const int32_t* selected,
                                const int32_t* selected_count, int32_t max_selected,
                                float sm_scale, void* out, int32_t out_dtype,
                                float* lse_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 4. The whole step                                                        */
/* ------------------------------------------------------------------------ */
/*
 * ls_score_select followed by ls_sparse_attn_decode (same definitions, same
 * results bit for bit: both take the same kernel code, chunking and merge
 * order for the same shapes). For requests of at most 8192 blocks the step
 * is ONE launch (the Vortex post fuses the operators of a decode step,
 * "Making it fast") spread over the whole chip: workgroups score chunks of
 * each pair's candidate blocks, the last chunk of a pair to finish ranks the
 * pair and publishes its selection, workgroups of at most 16 selected
 * blocks attend it (each waits for its pair's selection; every wait is on a
 * workgroup of lower index, which the hardware starts first) and the last of
 * them merges the pair's partial softmax states in split order. Scores,
 * selection and partial states go through the workspace with device-coherent
 * accesses. Longer requests run the split kernels of the two calls back to
 * back.
 *
 * Arguments: as ls_score_select (q, summaries, batch, p, selected,
 * selected_count) and ls_sparse_attn_decode (k_pool, v_pool with geometry
 * `pool`, sm_scale, out, out_dtype, lse_out); the summary pool shares the
 * K/V pool's num_pages, num_heads and head_dim.
 * new_page_ids, n_new_pages: optional (NULL, 0) device list of physical
 *   pages that filled at this step; the call also (re)builds their bf16
 *   summaries, exactly as ls_build_block_summaries would (as
 *   ls_build_block_bounds would with p->score_mode = LS_SCORE_BOUNDS; summaries are
 *   built when a block fills up -- Vortex post, "Why Long Generations Are
 *   Expensive"). On the one-launch path this runs in extra workgroups of the
 *   same launch, concurrently with the pairs, so it is only valid if no
 *   selection of this call reads those summaries: each listed page must be
 *   a forced block of its request in this call -- e.g. its last block, with
 *   p->n_recent >= 1 (checked). Otherwise call ls_build_block_summaries
 *   first.
 * workspace: >= ls_sparse_decode_step_workspace_size() bytes, 256-byte
 *   aligned (block scores, walk entries, split states); zero-filled before
 *   its first use, and every call leaves it zero; calls that run
 *   concurrently need separate workspaces.
 * Execution: the routes of ls_score_select and ls_sparse_attn_decode. One
 *   launch for at least 64 pairs of at most 4096 blocks (one workgroup per
 *   pair, the refresh in extra workgroups) and for fewer pairs of at most
 *   8192 blocks (pairs spread over many workgroups, hand-offs inside the
 *   launch); otherwise the planned route's three launches (scoring with the
 *   refresh, ranking, attention), with the same results as the two calls.
 * Supported: head_dim 64 or 128; GQA group 1, 2, 4 or 8 (other than 4:
 *   the summary refresh, scoring, top-k and split attention as separate
 *   launches); page_size 16; max_blocks <= 16384 (LS_SCORE_BOUNDS: group 4,
 *   max_blocks <= 8192 and num_pages < 2^26).
 */
size_t ls_sparse_decode_step_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks, int32_t max_selected);

ls_status ls_sparse_decode_step(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                void* summaries, const void* k_pool, const void* v_pool,
                                ls_pool pool, ls_batch batch, const ls_select_params* p,
                                int32_t* selected, int32_t* selected_count, float sm_scale,
                                void* out, int32_t out_dtype, float* lse_out,
                                const int32_t* new_page_ids, int32_t n_new_pages, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * The same step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument. Its scratch is a fixed device array inside the
 * library, ls_noalloc_scratch_bytes() bytes (32 MiB) per GPU, held until the
 * process ends; the call allocates and frees nothing. Shapes whose
 * ls_sparse_decode_step_workspace_size() exceeds that size are rejected with
 * LS_ERR_UNSUPPORTED. Each call clears the array's control words itself (one
 * small fill kernel on `stream` before the step). Every call on a GPU uses
 * that GPU's one array, so calls that overlap on one GPU (other streams,
 * other host threads) race and give unspecified results: serialise them.
 * Arguments, results and errors otherwise as ls_sparse_decode_step (the
 * same kernels, hence the same bits).
 */
size_t ls_noalloc_scratch_bytes(void);

ls_status ls_sparse_decode_step_noalloc(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                        void* summaries, const void* k_pool, const void* v_pool,
                                        ls_pool pool, ls_batch batch, const ls_select_params* p,
                                        int32_t* selected, int32_t* selected_count,
                                        float sm_scale, void* out, int32_t out_dtype,
                                        float* lse_out, const int32_t* new_page_ids,
                                        int32_t n_new_pages, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 5. Learned-indexer selection                                             */
/* ------------------------------------------------------------------------ */
/*
 * Score every unit u of request r with a learned indexer and keep the top-k
 * (LeanSparse, "Memory-Efficient Serving for Native Sparse-Attention LLMs",
 * Eq. 6, with the original keys in place of its compressed codes):
 *
 *   s_u = sum_{h < num_heads} head_weights[r][h] * max(0, sigma_u * (q[r][h] . key_u))
 *
 * (fp32 accumulation of exact products; bf16 q, fp8 or bf16 keys, 128 dims).
 * Units are:
 *   LS_SEL_TOKENS -- the cached tokens t < L of the request (key_u = the fp8
 *     indexer key of token t, sigma_u = key_scales[page][slot], 1 if
 *     key_scales is NULL); with a candidate list, only the tokens of the
 *     blocks cand_blocks[r][0 .. cand_counts[r]-1] (coarse-to-fine: the
 *     exact pass restricted to the blocks a coarse pass kept). No forced
 *     units. selected[r][0 .. cnt-1] = the first min(topk, #units) units under
 *     the order (s descending, token ascending), as TOKEN ids, ascending;
 *     remaining entries up to max_selected are -1.
 *   LS_SEL_BLOCKS -- the blocks (= pages) of the request, scored through
 *     their block-mean indexer key (built by ls_build_block_summaries from
 *     the fp8 keys and scales; sigma = 1). Forced and candidate blocks exactly
 *     as in ls_score_select (sink / recent blocks and the partial last block
 *     are forced, not ranked); ties go to the lowest block index.
 * The result is deterministic. Selection ties are decided on fp32 scores.
 *
 * q:            [batch][num_heads][128] bf16 (num_heads 16, 32 or 64).
 * head_weights: [batch][num_heads] fp32.
 * keys:         LS_SEL_TOKENS: fp8 e4m3fn indexer key pool [num_pages]
 *               [page_size][128] (key_pool.dtype LS_DTYPE_FP8_E4M3FN);
 *               LS_SEL_BLOCKS: bf16 block-mean keys [num_pages][128]
 *               (key_pool.dtype LS_DTYPE_BF16). key_pool.num_heads = 1,
 *               head_dim = 128, page_size 16, 32 or 64 (tokens per block).
 * key_scales:   tokens: NULL or [num_pages][page_size] fp32; blocks: NULL.
 * batch:        page table of the indexer pool (block = page).
 * cand_blocks:  tokens only, optional: [batch][cand_cap] ascending block
 *               indices with counts cand_counts[batch] (e.g. the selection
 *               of a LS_SEL_BLOCKS call); entries past the count are ignored.
 *               With p->candidates == LS_CAND_TOKENS the list holds TOKEN
 *               ids instead, strictly ascending, all in complete pages (e.g.
 *               the candidates of ls_pq_select), and the units are those
 *               tokens followed by the tokens of the request's partial last
 *               page (LeanSparse §5, "Retrieving and refining candidates":
 *               exact scores of the candidates and of the recent keys not
 *               yet encoded). A list that breaks this rule gives an
 *               unspecified selection (never an out-of-range access).
 * p:            host pointer. max_selected >= topk (tokens), or
 *               >= min(max_blocks, topk + n_sink + n_recent + 1) (blocks).
 * selected, selected_count: [batch][max_selected] int32, [batch] int32.
 * scores_out:   NULL, or [batch][ls_indexer_score_stride(granularity, U)]
 *               fp32 receiving s_u at unit u (tokens: unit = position in the
 *               token range or candidate list, u = c * page_size + slot for
 *               candidate c; blocks: unit = block index, candidates only).
 * workspace:    >= ls_indexer_select_workspace_size(batch, granularity, U)
 *               bytes, 256-byte aligned, need not be initialised; U = units
 *               per request at most: tokens max_blocks * page_size, or
 *               cand_cap * page_size with block candidates, or cand_cap +
 *               page_size with token candidates (<= 262144); blocks
 *               max_blocks (<= 16384).
 * Token mode is three launches: the scoring (each workgroup also leaves the
 * range of its scores); a histogram of the scores remapped into 4,096
 * buckets, linearly between the request's smallest and largest score; and a
 * pass that keeps every unit above the bucket b* holding the k-th score and
 * lists b*'s units, which the last workgroup of each request to finish the
 * pass ranks by their fp32 score (Vortex post, "Making it fast": a monotonic
 * remap of the scores spreads them over the buckets, so b* holds few units).
 * The bucket of score s is, in fp32 with each step rounded once,
 *   t = (s - mn) * (4096 / (mx - mn)),  bucket = min(4095, floor(t)),
 * with mn, mx the request's smallest and largest score; every bucket is 0
 * when mx - mn is not a positive finite number.
 * p->approx = 1 (tokens mode) is the approximate top-k of the same post (an
 * early exit that stops refining and fills the rest from the boundary
 * bucket): every unit whose bucket lies above b*, then units of b* in
 * ascending unit order until there are topk. Deterministic; it differs from
 * the exact top-k only inside b*.
 */
enum { LS_SEL_TOKENS = 0, LS_SEL_BLOCKS = 1 };
enum { LS_CAND_BLOCKS = 0, LS_CAND_TOKENS = 1 };

typedef struct ls_indexer_params {
  int32_t struct_size;   /* = sizeof(ls_indexer_params)                       */
  int32_t granularity;   /* LS_SEL_TOKENS or LS_SEL_BLOCKS                    */
  int32_t topk;          /* units chosen by score (forced blocks not counted) */
  int32_t n_sink;        /* blocks only: forced blocks 0 .. n_sink-1          */
  int32_t n_recent;      /* blocks only: forced last n_recent blocks          */
  int32_t max_selected;  /* row capacity of `selected`                        */
  int32_t candidates;    /* LS_CAND_BLOCKS or LS_CAND_TOKENS: what cand_blocks */
                         /* holds (tokens mode with a candidate list)         */
  int32_t approx;        /* tokens mode: 0 exact top-k; 1 approximate top-k */
                         /* (the boundary bucket filled in unit order, below) */
} ls_indexer_params;

/* Row stride (in floats) of scores_out for up to max_units units. */
int32_t ls_indexer_score_stride(int32_t granularity, int32_t max_units);

size_t ls_indexer_select_workspace_size(int32_t batch_size, int32_t granularity,
                                        int32_t max_units);

ls_status ls_indexer_select(const void* q, int32_t q_dtype, int32_t num_heads,
                            const float* head_weights, const void* keys, const float* key_scales,
                            ls_pool key_pool, ls_batch batch, const int32_t* cand_blocks,
                            const int32_t* cand_counts, int32_t cand_cap,
                            const ls_indexer_params* p, int32_t* selected,
                            int32_t* selected_count, float* scores_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 6. Sparse multi-head latent attention over selected tokens               */
/* ------------------------------------------------------------------------ */
/*
 * For every request r and query head h, attention over the latent rows c_t
 * of the selected tokens t < L (Vortex post, "Designing for a new
 * architecture": every query head attends one shared latent head whose rows
 * are both key -- all 576 entries, compressed content plus rope part -- and
 * value -- the first 512 entries):
 *   z_t = sm_scale * sum_{d<576} q[r][h][d] * c_t[d],
 *   out[r][h][:] = sum_t e^{z_t - M} c_t[0:512] / sum_t e^{z_t - M},
 *   lse_out[r][h] = M + ln sum_t e^{z_t - M}
 * fp32 logits, softmax and accumulation; the token set is split over
 * workgroups of 256 selected tokens whose partial states are merged by
 * log-sum-exp in split order (deterministic). Empty T: out = 0, lse = -inf.
 * Output rounded once (nearest-even) to out_dtype.
 *
 * q:        [batch][num_q_heads][576] bf16; num_q_heads a multiple of 32 (<= 256).
 * latent:   [num_pages][page_size][576] bf16 (pool.num_heads = 1,
 *           pool.head_dim = 576, pool.dtype = LS_DTYPE_BF16).
 * selected: [batch][max_selected] token ids (e.g. from ls_indexer_select),
 *           counts in selected_count[batch]; ids outside [0, L) are skipped.
 *           selected == NULL and selected_count == NULL attend every cached
 *           token (dense).
 * out:      [batch][num_q_heads][512] of out_dtype (bf16 or fp32).
 * lse_out:  NULL or [batch][num_q_heads] fp32.
 * workspace: >= ls_sparse_mla_decode_workspace_size(batch, num_q_heads,
 *           max_selected, or max_blocks * page_size when dense) bytes,
 *           256-byte aligned (split partial states); need not be initialised.
 */
int32_t ls_mla_num_splits(int32_t max_tokens);

size_t ls_sparse_mla_decode_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                           int32_t max_tokens);

ls_status ls_sparse_mla_decode(const void* q, int32_t q_dtype, int32_t num_q_heads,
                               const void* latent, ls_pool pool, ls_batch batch,
                               const int32_t* selected, const int32_t* selected_count,
                               int32_t max_selected, float sm_scale, void* out,
                               int32_t out_dtype, float* lse_out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 8. Sink + recent window attention, in place                               */
/* ------------------------------------------------------------------------ */
/*
 * The window baseline of the ByteCross paper ("Where Activation Sparsity and
 * KV-Cache Sparsity Cross in LLM Decoding", §4.1 and Appendix A, after
 * attention sinks): every query head attends, exactly, the tokens
 *   [0, ns) and [lo, L),  ns = min(n_sink, L),  lo = max(ns, L - window)
 * of its request, read where they are in the paged cache (no copy). The
 * paper runs the window and the sinks as two calls merged by log-sum-exp;
 * here both ranges are positions of one split-K call whose splits are merged
 * by the same log-sum-exp combine. A block holding both the last sinks and
 * the first window tokens is read twice with disjoint token ranges.
 * Arguments as in ls_sparse_attn_decode (no selection); n_sink, window >= 0;
 * pool.num_pages < 2^22. lse_out (optional) gets the natural-log LSE of the
 * logits over the attended tokens (-inf for an empty request, whose output
 * is 0). workspace: >= ls_window_attn_decode_workspace_size() bytes,
 * 256-byte aligned.
 */
size_t ls_window_attn_decode_workspace_size(int32_t batch_size, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_blocks, int32_t n_sink,
                                            int32_t window);
ls_status ls_window_attn_decode(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                const void* k_pool, const void* v_pool, ls_pool pool,
                                ls_batch batch, int32_t n_sink, int32_t window, float sm_scale,
                                void* out, int32_t out_dtype, float* lse_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 9. One-time SnapKV-style selection and gather                             */
/* ------------------------------------------------------------------------ */
/*
 * The scored KV selection of the ByteCross paper ("Where Activation Sparsity
 * and KV-Cache Sparsity Cross in LLM Decoding", §4.1 and Appendix A, "Scored
 * selection"), run once after prefill. For request r (L cached tokens) and
 * KV head g, the last n_obs prompt queries q_obs[r][w] (query w at position
 * L - n_obs + w, attending the positions up to its own) each give a softmax
 * over the cache with the logits sm_scale * q . k; the score of position t is
 * the sum of its probabilities over the n_obs queries and the group's 4
 * query heads (computed in fp32: per-row max and sum over 256-position
 * chunks, then the probabilities summed over the rows in a fixed order).
 * Scores are averaged over the 7 positions t-3 .. t+3 (zero outside the
 * prefix [0, L - n_obs), divisor 7). Kept: positions [0, min(n_sink, L -
 * n_obs)), the n_obs observation positions, and the prefix positions with
 * the largest averaged scores (ties to the lowest position) up to `budget`
 * in all (at most L).
 *
 * q_obs:    [batch][n_obs][num_q_heads][head_dim] bf16 (n_obs 1 .. 64,
 *           group size 4).
 * max_len:  >= every seq_len, <= 131072; batch * kv heads * max_len < 2^31.
 * selected: [batch][kv heads][budget] int32 positions, ascending, -1 after
 *           counts[batch][kv heads].
 * scores_out: NULL or [batch][kv heads][max_len] fp32 (the unaveraged score
 *           of every position < L, 0 after).
 * workspace: >= ls_snapkv_select_workspace_size() bytes, 256-byte aligned
 *           (includes the segmented radix sort's temporary storage).
 */
size_t ls_snapkv_select_workspace_size(int32_t batch_size, int32_t num_kv_heads,
                                       int32_t max_len);
ls_status ls_snapkv_select(const void* q_obs, int32_t q_dtype, int32_t num_q_heads,
                           int32_t n_obs, const void* k_pool, ls_pool pool, ls_batch batch,
                           int32_t max_len, float sm_scale, int32_t n_sink, int32_t budget,
                           int32_t* selected, int32_t* counts, float* scores_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The kept entries gathered once into contiguous buffers (the paper's
 * contiguous cache that every later decode step reads in one call):
 * k_out, v_out: [batch][kv heads][ceil(budget / 16) * 16][head_dim] bf16;
 * row i of (r, g) is position selected[r][g][i] for i < counts[r][g], zero
 * after. Reading it back with ls_sparse_attn_decode (no selection) works on
 * the view of batch * kv heads requests of one KV head each, 16-token pages
 * in order. */
ls_status ls_snapkv_gather(const void* k_pool, const void* v_pool, ls_pool pool, ls_batch batch,
                           const int32_t* selected, const int32_t* counts, int32_t budget,
                           void* k_out, void* v_out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* 7. PQ32 coarse scoring of indexer keys                                    */
/* ------------------------------------------------------------------------ */
/*
 * LeanSparse §5, "Approximate scoring with PQ": each 128-dim indexer key
 * x = scale * fp8 is cut into 32 subvectors of 4 dims and stored as 32
 * one-byte codes, code j = the nearest centroid of subvector j in codebook
 * C_j (256 centroids). The coarse score of a token replaces every subvector
 * by its centroid in the indexer score (Eq. 6):
 *   s~_t = sum_h head_weights[r][h] * max(0, sum_j q[r][h][4j..4j+3] . C_j[c_t,j]).
 * The C best tokens by s~ are candidates; ls_indexer_select with
 * LS_CAND_TOKENS then scores them and the partial last page's tokens
 * exactly and picks the final top-k ("Retrieving and refining candidates").
 *
 * codebooks: [32][256][4] bf16, 16-byte aligned.
 * codes:     [key_pool.num_pages][page_size][32] uint8, 8-byte aligned: the
 *            codes of token slot s of physical page p at codes[p][s].
 * key_pool:  the fp8 indexer key pool (dtype LS_DTYPE_FP8_E4M3FN, num_heads
 *            1, head_dim 128, page_size 16, 32 or 64).
 */

/* Codes of every token of the listed pages (pages as they fill). Nearest
 * centroid by squared Euclidean distance computed in float64 in the order
 * ((d0 d0 + d1 d1) + d2 d2) + d3 d3, d_t = x_t - c_t, each operation rounded
 * once; ties to the lowest centroid. Pages outside [0, num_pages) are
 * skipped. keys / key_scales as in ls_indexer_select (key_scales NULL: 1). */
ls_status ls_pq_encode(const void* keys, const float* key_scales, ls_pool key_pool,
                       const int32_t* page_ids, int32_t n_pages, const void* codebooks,
                       uint8_t* codes, hipStream_t stream);

/* Codebooks trained by k-means (Lloyd) on the tokens of the listed pages
 * (offline; token i = slot i % page_size of page_ids[i / page_size]).
 * Centroid c of subspace j starts as subvector j of token init_tokens[c]
 * (device int32 [256]; zero for an entry outside [0, n_pages * page_size)),
 * rounded to bf16; each of `iters` iterations encodes every token, then sets
 * each centroid with members to their mean and keeps the others. The mean
 * is order-independent: member values are summed as the integers
 * rint(v * 2^24) (64-bit), and (sum / count) * 2^-24 (float64) is rounded
 * once to bf16; sums must stay below 2^53 in magnitude (n_pages * page_size
 * * max |x| < 2^29). codebooks is written (it is the iteration state).
 * workspace: >= ls_pq_train_workspace_size() bytes, 256-byte aligned.
 * iters: 0 .. 1000. */
size_t ls_pq_train_workspace_size(void);
ls_status ls_pq_train(const void* keys, const float* key_scales, ls_pool key_pool,
                      const int32_t* page_ids, int32_t n_pages, const int32_t* init_tokens,
                      int32_t iters, void* codebooks, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Coarse selection: per request, the n_candidates tokens of the complete
 * pages with the largest s~ (ties to the lowest token), as token ids,
 * ascending, in candidates[r][0 .. counts[r]-1]; -1 after. q / head_weights
 * / batch as in ls_indexer_select. scores_out: NULL or
 * [batch][ls_indexer_score_stride(LS_SEL_TOKENS, max_blocks * page_size)]
 * fp32 (s~ at token t). workspace: >= ls_indexer_select_workspace_size(batch,
 * LS_SEL_TOKENS, max_blocks * page_size) bytes. Three launches: the coarse
 * scores, then the token top-k of ls_indexer_select (histogram of the
 * remapped scores, mark + finish). */
ls_status ls_pq_select(const void* q, int32_t q_dtype, int32_t num_heads,
                       const float* head_weights, const uint8_t* codes, const void* codebooks,
                       ls_pool key_pool, ls_batch batch, int32_t n_candidates,
                       int32_t* candidates, int32_t* candidate_counts, float* scores_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Miss filter before the exact rerank (LeanSparse §5, "Retrieving and
 * refining candidates"): of request r's candidates candidates[r][0 ..
 * counts[r]-1] (token ids, e.g. from ls_pq_select), every one whose original
 * indexer key is resident on the GPU is kept, and a miss is kept only when its
 * approximate score is at least
 *   theta = s_(j) - sd,   j = min(topk, n),
 * s_(j) the j-th largest approximate score of the n candidates and sd their
 * sample standard deviation (denominator n - 1; 0 for n < 2), computed in
 * float64 from the fp32 scores (a miss whose score equals theta is kept).
 * Only the kept misses need their keys fetched over the host link.
 * candidates, candidate_counts: [batch][cap] int32, [batch] int32 (counts
 *   clamped to [0, cap]); an entry outside [0, score_stride) is not a
 *   candidate (not counted, not kept). cap: 1 .. 4096.
 * scores:   [batch][score_stride] fp32, the approximate score at token t
 *   (ls_pq_select's scores_out, score_stride = its row stride).
 * resident: [batch][resident_words] uint32 bitmap, bit t % 32 of word t / 32
 *   set when token t's key is resident; tokens at or past 32 *
 *   resident_words are misses. May be NULL when resident_words is 0.
 * topk:     the final selection size k (>= 1).
 * kept, kept_counts: [batch][cap] int32 (the kept candidates in their
 *   input order, -1 after), [batch] int32. kept may be candidates itself.
 * misses_kept: NULL or [batch] int32, the number of kept misses.
 * One launch, one workgroup per request; deterministic (the float64 sums
 * are reduced in a fixed order). */
ls_status ls_pq_filter_misses(const int32_t* candidates, const int32_t* candidate_counts,
                              int32_t cap, const float* scores, int32_t score_stride,
                              const uint32_t* resident, int32_t resident_words,
                              int32_t batch_size, int32_t topk, int32_t* kept,
                              int32_t* kept_counts, int32_t* misses_kept, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Introspection                                                             */
/* ------------------------------------------------------------------------ */
/* Message for the last non-OK status returned on the calling thread ("" if
 * none). Host pointer owned by the library. */
const char* ls_last_error(void);

/* Library version and build string, e.g. "libls 0.2.0 abi 2 gfx950". */
const char* ls_version(void);

/* Measurement reference: one plain streaming read of `bytes` bytes at `src`
 * (every 16-byte word read once, non-temporal, many loads in flight), the
 * bandwidth this GPU delivers to a pure read, against which the decode
 * step's bandwidth is reported (ByteCross §4.4 and App. D price decode
 * kernels against the bandwidth the memory actually delivers). src: 16-byte
 * aligned, bytes a multiple of 16. sink: device, ls_stream_read_sink_words()
 * uint32 words, overwritten so that their XOR is the XOR of all 32-bit words
 * of the buffer (no load is dead, and the read can be checked). bytes == 0:
 * nothing is launched and sink is left as it was. Errors: LS_ERR_INVALID
 * for a null or misaligned pointer or a size not a multiple of 16. */
int32_t ls_stream_read_sink_words(void);
ls_status ls_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Debug check of a batch's device data                                      */
/* ------------------------------------------------------------------------ */
/* The kernels clamp device data that breaks the ls_batch contract (see
 * ls_batch); these calls report it. Violation kinds (bits): */
enum {
  LS_BATCH_BAD_INDPTR = 1,               /* page_indptr[r] < 0 or page_indptr[r+1] < page_indptr[r] */
  LS_BATCH_NEGATIVE_LENGTH = 2,          /* seq_lens[r] < 0                               */
  LS_BATCH_LENGTH_BEYOND_PAGES = 4,      /* ceil(seq_lens[r]/page_size) > pages in r's list */
  LS_BATCH_LENGTH_BEYOND_MAX_BLOCKS = 8, /* ceil(seq_lens[r]/page_size) > max_blocks       */
  LS_BATCH_PAGE_OUT_OF_RANGE = 16        /* a page id a kernel would read is outside [0, num_pages) */
};

/* Check `batch` against a pool of num_pages pages of page_size tokens: one
 * workgroup walks the requests and, per request, the page ids of the blocks
 * a kernel reads (below min(ceil(seq_lens[r]/page_size), list length,
 * max_blocks)); it reads only entries inside each request's list, so the
 * page list must hold page_indptr[batch_size] entries, as for every call.
 * report: device, 4 int32, overwritten on the stream: [0] the kinds found
 * (OR of the bits above), [1] the number of violating requests, [2] the
 * first violating request or -1, [3] the number of requests checked.
 * Errors: LS_ERR_INVALID for a null or misaligned report, a bad batch (as
 * every call) or page_size / num_pages < 1. batch_size 0 writes {0,0,-1,0}. */
ls_status ls_check_batch(ls_batch batch, int32_t page_size, int32_t num_pages, int32_t* report,
                         hipStream_t stream);

/* Debug mode (off by default; on when the environment holds LS_DEBUG set to
 * anything but "" or "0" when the library first looks, or after
 * ls_debug_enable(1)): every call that takes an ls_batch first enqueues the
 * same check on its stream, which adds into 4 words the library keeps per
 * GPU: [0] the kinds found (OR), [1] calls with a violation, [2] violating
 * requests, [3] calls checked. The check is one more kernel per call and
 * can be captured in a graph. */
void ls_debug_enable(int32_t on);
int32_t ls_debug_enabled(void);

/* Copy the current GPU's debug words to host_report (4 int32) and clear
 * them. Synchronises the device (not for use under stream capture).
 * Errors: LS_ERR_INVALID for a null host_report; LS_ERR_HIP. */
ls_status ls_debug_report(int32_t* host_report);

/* Number of split-K partitions ls_sparse_attn_decode uses for a given
 * selection capacity (max_selected, or max_blocks on the dense path). */
int32_t ls_attn_num_splits(int32_t max_selected);


#ifdef __cplusplus
}
#endif

#endif /* LS_H_ */

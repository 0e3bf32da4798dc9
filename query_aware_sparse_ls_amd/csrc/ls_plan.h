// The decode step planned from the lengths of the step (k_plan.hip):
// arguments, the grid and the workspace layout. Internal to libls.
//
// The work of a call is laid out flat -- the candidate summary tiles of
// every (request, kv head) pair in pair order, or the selected positions of
// every pair -- and cut into equal contiguous ranges, one per workgroup of a
// fixed grid, so that short and long requests cost the chip alike (Vortex
// post, "Making it fast": the work is planned at the start of each step from
// the sequence lengths, balancing workgroups across requests of different
// lengths). Every workgroup derives the plan itself from the lengths or
// counts on the device: nothing is read back to the host, and a call can be
// captured in a graph.
#pragma once

#include "ls_internal.h"

namespace ls {

constexpr int kPlanWaves = 4;
constexpr int kPlanThreads = kPlanWaves * kWave;   // scoring and attention workgroups
constexpr int kPlanRankThreads = 512;              // ranking workgroups (one per pair)
// Workgroups per call (measured on MI355X): scoring, four per CU; attention,
// two per CU with two K/V blocks in flight per wave.
#ifndef LS_PLAN_SCORE_GRID
#define LS_PLAN_SCORE_GRID 1024
#endif
#ifndef LS_PLAN_ATTN_GRID
#define LS_PLAN_ATTN_GRID 512
#endif
constexpr int kPlanScoreGrid = LS_PLAN_SCORE_GRID;   // scoring workgroups per call
constexpr int kPlanAttnGrid = LS_PLAN_ATTN_GRID;     // attention workgroups per call
constexpr int kPlanSubTiles = 16;                  // tiles per scoring pass (256 blocks)
constexpr int kPlanSubPositions = 64;              // positions per attention pass
constexpr int kPlanMaxBlocks = 16384;              // blocks per request
constexpr int kPlanCtlWords = 64;                  // control words ahead of the counters

// Scoring + ranking (ls_score_select), attention (ls_sparse_attn_decode).
struct PlanArgs {
  ScoreArgs sa;
  TopkArgs ta;
  AttnArgs aa;
  SummaryUpdate up;
  float* rows;          // [pairs][max_blocks] block scores (the caller's scores_out, or scratch)
  bool zero_rows;       // the ranker leaves the rows it read zero (scratch rows)
  int32_t* ents;        // step: [pairs][max_selected] walk entries the ranker writes
                        // beside the selection (page * 32 + tokens, -1: none), which
                        // the attention reads and resets to 0; null otherwise
  uint32_t* ctl;        // kPlanCtlWords words, then one arrival counter per pair
  float* slots;         // [2 * kPlanAttnGrid][4][D + 2] partial states of split pairs
  int32_t pairs;
  int32_t max_blocks;
};

inline size_t plan_align(size_t x) { return (x + 255) / 256 * 256; }
inline size_t plan_ctl_bytes(int pairs) {
  return plan_align(((size_t)kPlanCtlWords + (size_t)pairs) * sizeof(uint32_t));
}
inline size_t plan_rows_bytes(int pairs, int max_blocks) {
  return plan_align((size_t)pairs * max_blocks * sizeof(float));
}
inline size_t plan_slots_bytes(int head_dim) {
  return plan_align((size_t)2 * kPlanAttnGrid * 4 * (head_dim + 2) * sizeof(float));
}

// Shapes the planned kernels serve: GQA groups of 4, page = block = 16
// tokens, head_dim 64 or 128, at most kPlanMaxBlocks blocks per request,
// page ids below 2^26 (walk entries hold page * 32 + tokens), and fewer
// than 2^31 blocks over all pairs (the flat spaces are indexed in 32 bits).
inline bool plan_ok(int group, int head_dim, int max_blocks, int num_pages, int pairs) {
  return group == 4 && (head_dim == 64 || head_dim == 128) && max_blocks <= kPlanMaxBlocks &&
         num_pages < (1 << 26) && (long long)pairs * max_blocks < (1ll << 31);
}

// Summary refresh + scoring, then one ranking workgroup per pair.
hipError_t launch_plan_select(const PlanArgs& p, hipStream_t st);
// Attention over the selection (aa.selected), or over every block (dense).
hipError_t launch_plan_attend(const PlanArgs& p, hipStream_t st);

}  // namespace ls

// The decode step spread over many workgroups per (request, kv head) pair
// (k_flow.hip): arguments, the per-call plan and the workspace layout.
// Internal to libls.
#pragma once

#include "ls_internal.h"

namespace ls {

constexpr int kFlowWaves = 4;
constexpr int kFlowThreads = kFlowWaves * kWave;
constexpr int kFlowMaxChunks = 64;          // score chunks per pair
constexpr int kFlowMaxChunkBlocks = 256;    // blocks per score chunk (16 tiles)
constexpr int kFlowMaxSplit = 64;           // selection positions per attention split
constexpr int kFlowMaxBlocks = 8192;        // blocks per request
constexpr int kFlowSpinLimit = 1 << 20;     // polls of a hand-off before giving up

// Default chunk and split sizes (measured on MI355X).
#ifndef LS_FLOW_CHUNK_TILES
#define LS_FLOW_CHUNK_TILES 8               // 128 candidate blocks per score item
#endif
#ifndef LS_FLOW_SPLIT
#define LS_FLOW_SPLIT 16                    // selection positions per attention item (at most)
#endif

// Control words: ctl[kCtlError] is set when a hand-off wait gives up; then,
// from word kFlowCtlWords on, two arrival counters per pair (score chunks,
// attention splits).
constexpr int kFlowCtlWords = 64;
enum { kCtlError = 0 };

enum { kFlowStep = 0, kFlowSelect = 1, kFlowAttend = 2 };

// Every word handed over is reset to zero by its reader, so that the
// regions are zero between calls; walk entries are also polled (zero = not
// written yet).
struct FlowArgs {
  ScoreArgs sa;
  TopkArgs ta;
  AttnArgs aa;
  SummaryUpdate up;
  uint32_t* keys;       // [pairs][max_blocks] score keys (score_key)
  int32_t* ents;        // step: [pairs][max_selected] walk entries (-1: none)
  uint32_t* parts;      // [batch][Hq][splits][D + 2] split states (fp32 bits)
  uint32_t* ctl;        // kFlowCtlWords words, then [pairs][2] arrival counters
  float* scores_out;    // optional: the decoded block scores [pairs][max_blocks]
  int32_t pairs;
  int32_t max_blocks;
  int32_t chunks, chunk_tiles;   // score items per pair, 16-block tiles per item
  int32_t splits, split;         // attention items per pair, positions per item
  int32_t n_refresh;             // refresh items (kFlowWaves tiles each)
};

struct FlowPlan {
  int chunks, chunk_tiles, splits, split;
};

// Chunking of one call: score items of LS_FLOW_CHUNK_TILES tiles (halved
// when the batch has few pairs, so that the chip still gets ~512 items), at
// most kFlowMaxChunks per pair; attention items of at most LS_FLOW_SPLIT
// positions, sized evenly.
inline FlowPlan flow_plan(int pairs, int max_blocks, int max_selected) {
  FlowPlan p;
  const int ntiles = (max_blocks + 15) / 16;
  int ct = LS_FLOW_CHUNK_TILES;
  if ((long long)pairs * ((ntiles + ct - 1) / ct) < 512 && ct > 4) ct = 4;
  while ((ntiles + ct - 1) / ct > kFlowMaxChunks) ct *= 2;
  p.chunk_tiles = ct;
  p.chunks = (ntiles + ct - 1) / ct;
  if (p.chunks < 1) p.chunks = 1;
  const int ms = max_selected > 0 ? max_selected : 1;
  p.splits = (ms + LS_FLOW_SPLIT - 1) / LS_FLOW_SPLIT;
  p.split = (ms + p.splits - 1) / p.splits;
  return p;
}

inline size_t flow_align(size_t x) { return (x + 255) / 256 * 256; }

inline size_t flow_ctl_bytes(int pairs) {
  return flow_align(((size_t)kFlowCtlWords + 2 * (size_t)pairs) * sizeof(uint32_t));
}
inline size_t flow_keys_bytes(int pairs, int max_blocks) {
  return flow_align((size_t)pairs * max_blocks * sizeof(uint32_t));
}
inline size_t flow_ents_bytes(int pairs, int max_selected) {
  return flow_align((size_t)pairs * max_selected * sizeof(int32_t));
}
inline size_t flow_parts_bytes(int pairs, int head_dim, int splits) {
  return flow_align((size_t)pairs * 4 * splits * (head_dim + 2) * sizeof(uint32_t));
}

// Shapes the flow kernel serves: GQA groups of 4, page = block = 16 tokens,
// head_dim 64 or 128, at most kFlowMaxBlocks blocks per request, page ids
// below 2^26 (walk entries hold page * 32 + tokens).
inline bool flow_ok(int group, int head_dim, int max_blocks, int num_pages) {
  return group == 4 && (head_dim == 64 || head_dim == 128) && max_blocks <= kFlowMaxBlocks &&
         num_pages < (1 << 26);
}

hipError_t launch_flow(const FlowArgs& f, int mode, hipStream_t st);
// Zero n bytes (a multiple of 4) at p: the split and dense paths leave the
// workspace as they found it, zero.
hipError_t launch_zero(void* p, size_t n, hipStream_t st);

}  // namespace ls

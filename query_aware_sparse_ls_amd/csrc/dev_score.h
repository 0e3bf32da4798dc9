// GQA block scoring, wave-level device code (used by the standalone scoring
// kernel and by the fused decode-step kernel).
//
// s[r][g][j] = agg_{h in group g} q[r][h] . summary[page(r,j)][g]
// (Vortex post: s_j = q . k̄_j, "Why Long Generations Are Expensive"; the
// vFlow block-top-k listing reduces the per-head block scores over the head
// axis before top-k, "Writing an algorithm: vFlow").
//
// Memory walk: a physical page's summaries for all KV heads are one
// contiguous run of Hkv * D * 2 bytes. Each lane loads 16 bytes (8 dims of one
// KV head's row), so a wave instruction reads 1 KB, coalesced within a page.
// A lane's (page offset, head, dim chunk) is the same for every page it
// visits, so the group's query values stay in registers as bf16 pairs and
// each chunk is consumed with v_dot2 (two exact bf16 products accumulated in
// fp32). A wave first loads the page ids of its pages (one hop), then issues
// every summary load at once (one hop), then computes: two dependent memory
// latencies per wave, many waves per CU. The D/8 lanes of a row are summed
// with DPP adds, then the group's heads are aggregated (max or mean).
#pragma once

#include "ls_internal.h"

namespace ls {

template <int D, int HKV, int G>
struct ScoreShape {
  static constexpr int kUnitsPerPage = HKV * D / 8;  // 16-byte units per page
  static constexpr int kLanesPerRow = D / 8;
  static constexpr int J = kUnitsPerPage >= kWave ? kUnitsPerPage / kWave : 1;   // loads/page
  static constexpr int PPI = kUnitsPerPage >= kWave ? 1 : kWave / kUnitsPerPage;  // pages/load
  static constexpr int NI = J >= 16 ? 1 : 16 / J;        // load rounds per wave (16 loads)
  static constexpr int kBlocksPerWave = NI * PPI;
  static_assert(kUnitsPerPage % kWave == 0 || kWave % kUnitsPerPage == 0, "page geometry");
};

__device__ __forceinline__ float dot8_bf16(const uint32_t* q, uint4 s, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[0]),
                                        __builtin_bit_cast(bf16x2_t, s.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[1]),
                                        __builtin_bit_cast(bf16x2_t, s.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[2]),
                                        __builtin_bit_cast(bf16x2_t, s.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[3]),
                                        __builtin_bit_cast(bf16x2_t, s.w), acc, false);
  return acc;
}

// Per-wave LDS staging of the scores, written out as contiguous runs.
template <int D, int HKV, int G>
struct ScoreLds {
  float s[HKV * ScoreShape<D, HKV, G>::kBlocksPerWave];
};

// One wave scores the candidate blocks of request r that fall in
// [wb0, wb0 + kBlocksPerWave). geo: the request's geometry. kDev: write the
// scores device-coherently (consumed by other workgroups of the same launch).
template <int D, int HKV, int G, bool kDev>
__device__ __forceinline__ void score_wave(const ScoreArgs& a, int r, const ReqGeom& geo,
                                           int wb0, int lane, ScoreLds<D, HKV, G>& st) {
  using S = ScoreShape<D, HKV, G>;
  constexpr int J = S::J, PPI = S::PPI, NI = S::NI, LPR = S::kLanesPerRow;
  const int lo = max(geo.c0, wb0), hi = min(geo.c1, wb0 + S::kBlocksPerWave);
  if (lo >= hi) return;
  int poff[J], gh[J], ch[J];
  uint32_t qv[J][G][4];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int u = j * kWave + lane;
    poff[j] = u / S::kUnitsPerPage;
    const int w = u % S::kUnitsPerPage;
    gh[j] = w / LPR;
    ch[j] = w % LPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 t = ldg16(a.q + ((size_t)r * (HKV * G) + gh[j] * G + h) * D + ch[j] * 8);
      qv[j][h][0] = t.x; qv[j][h][1] = t.y; qv[j][h][2] = t.z; qv[j][h][3] = t.w;
    }
  }
  const int32_t* pages = a.b.indices + geo.page_base;
  int blk[NI][J], pg[NI][J];
  bool ok[NI][J];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int b = wb0 + it * PPI + poff[j];
      const bool v = b >= lo && b < hi;
      blk[it][j] = b;
      pg[it][j] = v ? pages[b] : -1;
    }
  }
  uint4 buf[NI][J];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int p = pg[it][j];
      const bool v = p >= 0 && p < a.b.num_pages;
      ok[it][j] = v;
      buf[it][j] = v ? ldg16(a.summaries + ((size_t)p * HKV + gh[j]) * D + ch[j] * 8)
                     : make_uint4(0, 0, 0, 0);
    }
  }
  constexpr int BPW = S::kBlocksPerWave;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float s;
      {
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = group_sum<LPR>(dot8_bf16(qv[j][h], buf[it][j], 0.0f));
        s = part[0];
        if (a.group_agg == LS_AGG_MEAN) {
#pragma unroll
          for (int h = 1; h < G; ++h) s += part[h];
          s *= (1.0f / G);
        } else {
#pragma unroll
          for (int h = 1; h < G; ++h) s = fmaxf(s, part[h]);
        }
      }
      if (ch[j] == 0) st.s[gh[j] * BPW + it * PPI + poff[j]] = s;
    }
  }
  wave_lds_sync();
  // scores[r][g][wb0 .. wb0 + BPW): runs of BPW consecutive floats per head
  float* out = a.scores + (size_t)r * HKV * a.b.max_blocks;
  for (int i = lane; i < HKV * BPW; i += kWave) {
    const int g = i / BPW, b = wb0 + i % BPW;
    if (b >= lo && b < hi) st_x<kDev>(&out[(size_t)g * a.b.max_blocks + b], st.s[i]);
  }
  wave_lds_sync();
}

}  // namespace ls

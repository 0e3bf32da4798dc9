// GQA block scoring: s[r][g][j] = agg_{h in group g} q[r][h] . summary[page(r,j)][g]
//
// Vortex post, "Why Long Generations Are Expensive" (s_j = q . k̄_j) and the
// vFlow block-top-k listing ("Writing an algorithm: vFlow"), where the block
// scores of all query heads are reduced over the head axis before top-k.
//
// Memory walk: a physical page's summaries for all KV heads are one
// contiguous run of Hkv * D * 2 bytes, so the kernel streams whole pages: a
// wave's 64 lanes each load 16 bytes (8 dims of one KV head's summary row),
// i.e. 1 KB per wave instruction, coalesced within each page. A lane's
// (head, dim-chunk) is fixed across pages, so the group's query values stay
// in registers as bf16 pairs, and each 16-byte chunk is consumed with
// v_dot2 (two bf16 products accumulated in fp32). The D/8 lanes that share a
// row are then reduced with xor-shuffles and the group's heads aggregated.
// Only candidate blocks (complete, neither sink nor recent) are read.
#include "ls_internal.h"

namespace ls {

template <int D, int HKV, int G>
struct ScoreShape {
  static constexpr int kUnitsPerPage = HKV * D / 8;       // 16-byte units per page
  static constexpr int kLanesPerRow = D / 8;
  static constexpr int kLoadsPerPage = kUnitsPerPage >= kWave ? kUnitsPerPage / kWave : 1;
  static constexpr int kPagesPerIter = kUnitsPerPage >= kWave ? 1 : kWave / kUnitsPerPage;
  static_assert(kUnitsPerPage % kWave == 0 || kWave % kUnitsPerPage == 0, "page size");
};

constexpr int kScoreBlocksPerWG = 64;
constexpr int kScoreUnroll = 4;

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

template <int D, int HKV, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  using S = ScoreShape<D, HKV, G>;
  constexpr int J = S::kLoadsPerPage, PPI = S::kPagesPerIter, LPR = S::kLanesPerRow;
  const int r = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
  const int blk0 = blockIdx.x * kScoreBlocksPerWG;
  const int lo = max(geo.c0, blk0), hi = min(geo.c1, blk0 + kScoreBlocksPerWG);
  if (lo >= hi) return;

  // this lane's fixed (page offset, kv head, dim chunk) for each load slot
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
  const size_t row_stride = (size_t)a.b.max_blocks;
  float* out = a.scores + (size_t)r * HKV * row_stride;
  // page groups of this workgroup, dealt round-robin to its 4 waves
  const int ngroups = (kScoreBlocksPerWG + PPI - 1) / PPI;
  for (int g0 = wave; g0 < ngroups; g0 += 4 * kScoreUnroll) {
    uint4 buf[kScoreUnroll][J];
    int blk[kScoreUnroll][J];
    bool ok[kScoreUnroll][J];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int b = blk0 + (g0 + 4 * u) * PPI + poff[j];
        bool v = (g0 + 4 * u) < ngroups && b >= lo && b < hi;
        int p = v ? pages[b] : 0;
        v = v && p >= 0 && p < a.b.num_pages;
        blk[u][j] = b;
        ok[u][j] = v;
        buf[u][j] = v ? ldg16(a.summaries + ((size_t)p * HKV + gh[j]) * D + ch[j] * 8)
                      : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = dot8_bf16(qv[j][h], buf[u][j], 0.0f);
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) {
#pragma unroll
          for (int h = 0; h < G; ++h) part[h] += __shfl_xor(part[h], o, kWave);
        }
        float s = part[0];
        if (a.group_agg == LS_AGG_MEAN) {
#pragma unroll
          for (int h = 1; h < G; ++h) s += part[h];
          s *= (1.0f / G);
        } else {
#pragma unroll
          for (int h = 1; h < G; ++h) s = fmaxf(s, part[h]);
        }
        if (ok[u][j] && ch[j] == 0) out[(size_t)gh[j] * row_stride + blk[u][j]] = s;
      }
    }
  }
}

template <int D, int HKV, int G>
static hipError_t launch(const ScoreArgs& a, hipStream_t st) {
  dim3 grid((a.b.max_blocks + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG, a.b.batch);
  hipLaunchKernelGGL((score_kernel<D, HKV, G>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  const int D = a.head_dim, H = a.num_kv_heads;
  if (D == 128) {
    switch (H) {
      case 1: return launch<128, 1, 4>(a, st);
      case 2: return launch<128, 2, 4>(a, st);
      case 4: return launch<128, 4, 4>(a, st);
      case 8: return launch<128, 8, 4>(a, st);
      case 16: return launch<128, 16, 4>(a, st);
    }
  } else {
    switch (H) {
      case 1: return launch<64, 1, 4>(a, st);
      case 2: return launch<64, 2, 4>(a, st);
      case 4: return launch<64, 4, 4>(a, st);
      case 8: return launch<64, 8, 4>(a, st);
      case 16: return launch<64, 16, 4>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ls

// Split-K gather attention over the selected blocks of a paged KV cache and
// the log-sum-exp merge of the splits (workgroup-level device code shared by
// the standalone attention kernels and the fused decode-step kernel).
//
// Vortex post, block top-k equation: o = softmax(q K_I^T / sqrt(d)) V_I over
// the tokens of the selected blocks I. The split results are merged by
// log-sum-exp, the merge the ByteCross paper ("Where Activation Sparsity and
// KV-Cache Sparsity Cross in LLM Decoding", App. A) applies to attention over
// disjoint token sets.
//
// A split is the run of at most CH consecutive positions of one (request, kv
// head) selection row. A (page, head) tile is page_size x D contiguous bf16.
// Thread t owns 8 dims of one token row of every block of the split; a wave
// instruction reads 1 KB contiguous and the workgroup a whole 4 KB tile. All
// K and V loads of the split are issued before any is used; there is no reuse
// of K/V across threads, so the data goes straight to registers.
//
// Each group of D/8 lanes owns one token row: the G query heads' logits are
// v_dot2 partial sums summed over those lanes with DPP adds, pre-scaled by
// sm_scale * log2 e so that each exponential is one exp2.
#pragma once

#include "ls_internal.h"

namespace ls {


template <int D, int G>
struct AttnShape {
  static constexpr int P = 16;            // tokens per block
  static constexpr int LPR = D / 8;       // lanes per token row
  static constexpr int RPW = kWave / LPR; // rows per wave
  static constexpr int ROWS = 4 * RPW;    // rows per workgroup round
  static constexpr int BPR = ROWS / P;    // blocks per round
};

template <int D, int G>
struct AttnLds {
  float acc[4][G][D];   // per-wave sums
  float m[4][G];
  float l[4][G];
};

__device__ __forceinline__ float dot8(const uint32_t* q, uint4 s, float acc) {
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

// Attention of kv group g of request r over the entries of split s: the
// positions [s*CH, s*CH + CH) of the (r, g) selection row (of the block list
// itself on the dense path), written as split s of the partial buffer:
// partials[r][g*G + h][s][0..D-1] = o relative to the split maximum m,
// [D] = m (log2 domain), [D+1] = l. Must be called by all 256 threads.
//
// Memory hops: (1) q, the selection count and the split's selection entries,
// all independent; (2) the page table; (3) K and V of every entry, all issued
// before any is used.
//
// Softmax: one maximum per head over the whole split (lane, DPP within the
// wave, LDS across the 4 waves), then p = 2^(z - m) and the sums over rows by
// lane-pair exchanges within a wave and LDS across waves, in a fixed order.
template <int D, int G, int CH, bool kDev>
__device__ __forceinline__ void attn_split(const AttnArgs& a, const ReqGeom& geo, int r, int g,
                                           int s, AttnLds<D, G>& sh) {
  using S = AttnShape<D, G>;
  constexpr int P = S::P, LPR = S::LPR, RPW = S::RPW, BPR = S::BPR;
  static_assert(CH % BPR == 0, "split length must be whole rounds");
  constexpr int NR = CH / BPR;  // rounds: one block per BPR rows
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = wave * RPW + lane / LPR;
  const int c = lane % LPR;
  const int bir = row / P, slot = row % P;
  const int HKV = a.num_kv_heads;
  const size_t item = (size_t)r * HKV + g;

  // hop 1
  uint32_t qv[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = ldg16(a.q + ((size_t)r * a.num_q_heads + g * G + h) * D + c * 8);
    qv[h][0] = t.x; qv[h][1] = t.y; qv[h][2] = t.z; qv[h][3] = t.w;
  }
  const bool sparse = a.selected != nullptr;
  const int npos = sparse ? a.max_selected : geo.nb;   // positions that exist
  int cnt = sparse ? ld_x<kDev>(&a.selected_count[item]) : geo.nb;
  const int32_t* srow = sparse ? a.selected + item * a.max_selected : nullptr;
  int blk[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int pos = s * CH + i * BPR + bir;
    blk[i] = pos < npos ? (sparse ? ld_x<kDev>(&srow[pos]) : pos) : -1;
  }
  cnt = cnt < 0 ? 0 : (cnt > npos ? npos : cnt);
  bool ok[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int pos = s * CH + i * BPR + bir;
    const int b = blk[i];
    ok[i] = pos < cnt && b >= 0 && b < geo.nb && b * P + slot < geo.L;
  }
  // hop 2: page table
  const int32_t* pages = a.b.indices + geo.page_base;
  int page[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) page[i] = ok[i] ? pages[blk[i]] : -1;
  // hop 3
  uint4 kr[NR], vr[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    ok[i] = ok[i] && page[i] >= 0 && page[i] < a.b.num_pages;
    const size_t off = (((size_t)(ok[i] ? page[i] : 0) * HKV + g) * P + slot) * D + c * 8;
    kr[i] = ok[i] ? ldg16(a.k_pool + off) : make_uint4(0, 0, 0, 0);
    vr[i] = ok[i] ? ldg16(a.v_pool + off) : make_uint4(0, 0, 0, 0);
  }

  float z[NR][G];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      z[i][h] = ok[i] ? group_sum<LPR>(dot8(qv[h], kr[i], 0.0f)) * a.sm_scale_log2 : kNegInf;
  }
  // split maximum per head
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < NR; ++i) mx = fmaxf(mx, z[i][h]);
    mx = wave_max_fast(mx);
    if (lane == 0) sh.m[wave][h] = mx;
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    M[h] = fmaxf(fmaxf(sh.m[0][h], sh.m[1][h]), fmaxf(sh.m[2][h], sh.m[3][h]));
  float l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.0f;
    if (M[h] != kNegInf) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float p = ok[i] ? exp2_fast(z[i][h] - M[h]) : 0.0f;
        l[h] += p;
        const uint4 v = vr[i];
        acc[h][0] += p * bf16_lo(v.x); acc[h][1] += p * bf16_hi(v.x);
        acc[h][2] += p * bf16_lo(v.y); acc[h][3] += p * bf16_hi(v.y);
        acc[h][4] += p * bf16_lo(v.z); acc[h][5] += p * bf16_hi(v.z);
        acc[h][6] += p * bf16_lo(v.w); acc[h][7] += p * bf16_hi(v.w);
      }
    }
  }
  // sum over the RPW rows of the wave (lanes that differ in the row bits),
  // by lane-pair exchanges in a fixed order
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if constexpr (LPR <= 8) {
      l[h] = xor_pair_sum<8>(l[h]);
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] = xor_pair_sum<8>(acc[h][d]);
    }
    l[h] = xor_pair_sum<32>(xor_pair_sum<16>(l[h]));
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = xor_pair_sum<32>(xor_pair_sum<16>(acc[h][d]));
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&sh.acc[wave][h][c * 8]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      if (c == 0) sh.l[wave][h] = l[h];
    }
  }
  __syncthreads();
  const int S_ = a.num_splits;
  float* part = a.partials + (((size_t)r * a.num_q_heads + g * G) * S_ + s) * (D + 2);
  for (int o = tid; o < G * D; o += 256) {
    const int h = o / D, d = o % D;
    const float O = ((sh.acc[0][h][d] + sh.acc[1][h][d]) + sh.acc[2][h][d]) + sh.acc[3][h][d];
    float* ph = part + (size_t)h * S_ * (D + 2);
    st_x<kDev>(&ph[d], O);
    if (d == 0) {
      const float Ls = ((sh.l[0][h] + sh.l[1][h]) + sh.l[2][h]) + sh.l[3][h];
      st_x<kDev>(&ph[D], M[h]);
      st_x<kDev>(&ph[D + 1], Ls);
    }
  }
  __syncthreads();
}

// Merge the S partials of query head `item` (= r * Hq + h) in split order and
// write the rounded output and lse. One wave; lane owns dims lane + 64 j.
template <int D, bool kDev>
__device__ __forceinline__ void combine_head(const AttnArgs& a, int item, int lane) {
  constexpr int DPL = D / kWave;
  const int S = a.num_splits;
  const float* part = a.partials + (size_t)item * S * (D + 2);
  // every split's (m, l), 64 splits per pass, then the maximum
  float M = kNegInf;
  for (int s0 = 0; s0 < S; s0 += kWave) {
    const int s = s0 + lane;
    const float ms = s < S ? ld_x<kDev>(&part[(size_t)s * (D + 2) + D]) : kNegInf;
    M = fmaxf(M, wave_max(ms));
  }
  float O[DPL], Ls = 0.0f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) O[j] = 0.0f;
  if (M != kNegInf) {
    constexpr int U = 8;  // splits loaded per batch, all loads in flight
    for (int s0 = 0; s0 < S; s0 += U) {
      float ms[U], ls[U], os[U][DPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u;
        const float* ps = part + (size_t)(s < S ? s : 0) * (D + 2);
        ms[u] = s < S ? ld_x<kDev>(&ps[D]) : kNegInf;
        ls[u] = ld_x<kDev>(&ps[D + 1]);
#pragma unroll
        for (int j = 0; j < DPL; ++j) os[u][j] = ld_x<kDev>(&ps[lane + j * kWave]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float e = exp2_fast(ms[u] - M);   // 0 for absent / empty splits
        Ls += e * ls[u];
#pragma unroll
        for (int j = 0; j < DPL; ++j) O[j] += e * os[u][j];
      }
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    const float o = O[j] * inv;
    const size_t idx = (size_t)item * D + lane + j * kWave;
    if (a.out_dtype == LS_DTYPE_FP32) reinterpret_cast<float*>(a.out)[idx] = o;
    else reinterpret_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_rne(o);
  }
  if (a.lse && lane == 0)
    a.lse[item] = (M == kNegInf || !(Ls > 0.0f)) ? kNegInf : (M + log2f(Ls)) * kLn2;
}

}  // namespace ls

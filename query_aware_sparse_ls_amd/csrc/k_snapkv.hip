// One-time SnapKV-style selection and gather (ByteCross paper, §4.1 and
// Appendix A, "Scored selection"): after prefill, the last W prompt queries
// (observation window; query w sits at position L - W + w and attends the
// positions up to its own) each give a softmax over the cache of their KV
// head; a position's score is the sum of its probabilities over the W
// queries and the group's query heads; scores are averaged over 7 positions
// (zero outside the prefix [0, L - W)); the first n_sink positions and the W
// observation positions are kept, and the rest of the budget goes to the
// prefix positions with the largest averaged score (ties to the lowest
// position). The kept keys and values are then gathered into a contiguous
// buffer per (request, KV head), which a decode step reads in one call.
//
// Kernels (all per (request, KV head) pair; one thread per cache position in
// chunks of 256 positions, the pair's W x G query rows in LDS):
//   snap_stats_kernel   per row and chunk: max and sum of exp of the logits;
//   snap_rowstat_kernel per row: the max and 1 / sum over all chunks;
//   snap_score_kernel   per position: sum over rows of exp(z - max) / sum
//                       (rows in a fixed order: deterministic);
//   snap_pool_kernel    width-7 average, sort keys of the candidates;
//   (segmented radix sort of the candidates by averaged score, descending,
//    stable: equal scores keep ascending positions)
//   snap_emit_kernel    forced positions + the first k sorted, ascending;
//   snap_gather_kernel  K and V rows of the kept positions, contiguous.
// This runs once per prompt, not per decode step; the dot products are
// plain fp32 VALU work (about 0.3 TFLOP at 16 x 32K).
#include <hipcub/hipcub.hpp>

#include "ls_internal.h"

namespace ls {

constexpr int kSnapChunk = 256;   // positions per workgroup (one per thread)
constexpr int kSnapRows = kSnapMaxObs * 4;

// Logit (scaled) of row `row` (= w * 4 + h) for the key held in k[] (fp32).
template <int D>
__device__ __forceinline__ float snap_dot(const uint16_t* q_lds, int row, const float* k) {
  const uint32_t* qr = reinterpret_cast<const uint32_t*>(q_lds + (size_t)row * D);
  float acc = 0.0f;
#pragma unroll
  for (int d = 0; d < D / 2; ++d) {
    const uint32_t w = qr[d];
    acc = fmaf(__uint_as_float(w << 16), k[2 * d], acc);
    acc = fmaf(__uint_as_float(w & 0xffff0000u), k[2 * d + 1], acc);
  }
  return acc;
}

// The pair's W x 4 query rows into LDS (row w * 4 + h, head g * 4 + h) and
// this thread's key (position p) into registers; returns whether p < L.
template <int D>
__device__ __forceinline__ bool snap_setup(const SnapArgs& a, int r, int g, int p, const ReqGeom& geo,
                                           uint16_t* q_lds, float* k) {
  const int rows = a.n_obs * 4;
  const int tid = threadIdx.x;
  for (int i = tid; i < rows * D / 8; i += kSnapChunk) {
    const int row = i / (D / 8), c = i % (D / 8);
    const int w = row / 4, h = row % 4;
    const uint4 v = *reinterpret_cast<const uint4*>(
        a.q_obs + (((size_t)r * a.n_obs + w) * a.num_q_heads + g * 4 + h) * D + 8 * c);
    *reinterpret_cast<uint4*>(q_lds + (size_t)row * D + 8 * c) = v;
  }
  const bool valid = p < (geo.L < a.max_len ? geo.L : a.max_len);
  const int blk = p / 16;
  int page = valid && blk < geo.nb ? a.b.indices[geo.page_base + blk] : -1;
  if (page < 0 || page >= a.b.num_pages) page = -1;
  const uint16_t* kr = a.k_pool + (((size_t)(uint32_t)(page >= 0 ? page : 0) * a.num_kv_heads + g) * 16 +
                                   (p & 15)) * D;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const uint4 v = page >= 0 ? *reinterpret_cast<const uint4*>(kr + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      k[8 * c + 2 * j] = __uint_as_float(w4[j] << 16);
      k[8 * c + 2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
    }
  }
  return valid && page >= 0;
}

template <int D>
__global__ __launch_bounds__(kSnapChunk) void snap_stats_kernel(SnapArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kSnapRows * D];
  __shared__ float red_m[kSnapChunk / kWave][kSnapRows], red_s[kSnapChunk / kWave][kSnapRows];
  const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const int p = c * kSnapChunk + tid;
  const int Lc = geo.L < a.max_len ? geo.L : a.max_len;   // positions past max_len are not read
  float k[D];
  const bool valid = snap_setup<D>(a, r, g, p, geo, q_lds, k);
  __syncthreads();
  const int rows = a.n_obs * 4;
  for (int row = 0; row < rows; ++row) {
    const int w = row / 4;
    const bool ok = valid && p <= Lc - a.n_obs + w;   // causal
    const float z = ok ? snap_dot<D>(q_lds, row, k) * a.sm_scale_log2 : -__builtin_huge_valf();
    const float m = wave_max_fast(z);
    const float e = m == -__builtin_huge_valf() ? 0.0f : exp2f(z - m);
    const float sm = wave_sum(e);
    if (lane == 0) {
      red_m[wave][row] = m;
      red_s[wave][row] = sm;
    }
  }
  __syncthreads();
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  for (int row = tid; row < rows; row += kSnapChunk) {
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kSnapChunk / kWave; ++w) m = fmaxf(m, red_m[w][row]);
    float s = 0.0f;
    if (m != -__builtin_huge_valf()) {
#pragma unroll
      for (int w = 0; w < kSnapChunk / kWave; ++w) s += red_s[w][row] * exp2f(red_m[w][row] - m);
    }
    float* st = a.stats + ((pair * a.n_chunks + c) * kSnapRows + row) * 2;
    st[0] = m;
    st[1] = s;
  }
}

__global__ __launch_bounds__(kSnapRows) void snap_rowstat_kernel(SnapArgs a) {
  const size_t pair = blockIdx.x;
  const int row = threadIdx.x;
  if (row >= a.n_obs * 4) return;
  float m = -__builtin_huge_valf();
  for (int c = 0; c < a.n_chunks; ++c) m = fmaxf(m, a.stats[((pair * a.n_chunks + c) * kSnapRows + row) * 2]);
  float s = 0.0f;
  if (m != -__builtin_huge_valf())
    for (int c = 0; c < a.n_chunks; ++c) {
      const float* st = a.stats + ((pair * a.n_chunks + c) * kSnapRows + row) * 2;
      s += st[1] * exp2f(st[0] - m);
    }
  float* o = a.rowstat + (pair * kSnapRows + row) * 2;
  o[0] = m;
  o[1] = s > 0.0f ? 1.0f / s : 0.0f;
}

template <int D>
__global__ __launch_bounds__(kSnapChunk) void snap_score_kernel(SnapArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kSnapRows * D];
  __shared__ float rm[kSnapRows], rinv[kSnapRows];
  const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const int p = c * kSnapChunk + tid;
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int Lc = geo.L < a.max_len ? geo.L : a.max_len;
  float k[D];
  const bool valid = snap_setup<D>(a, r, g, p, geo, q_lds, k);
  const int rows = a.n_obs * 4;
  for (int row = tid; row < rows; row += kSnapChunk) {
    rm[row] = a.rowstat[(pair * kSnapRows + row) * 2];
    rinv[row] = a.rowstat[(pair * kSnapRows + row) * 2 + 1];
  }
  __syncthreads();
  float score = 0.0f;
  for (int row = 0; row < rows; ++row) {
    const int w = row / 4;
    if (valid && p <= Lc - a.n_obs + w) {
      const float z = snap_dot<D>(q_lds, row, k) * a.sm_scale_log2;
      score += exp2f(z - rm[row]) * rinv[row];
    }
  }
  if (p < a.max_len) a.scores[pair * a.max_len + p] = p < Lc ? score : 0.0f;
}

// Averaged scores of the candidates [n_sink, L - W) as sort keys (values:
// positions), segment `pair` at [pair * max_len, + count).
__global__ __launch_bounds__(256) void snap_pool_kernel(SnapArgs a) {
  const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int Lc = geo.L < a.max_len ? geo.L : a.max_len;
  const int npre = Lc > a.n_obs ? Lc - a.n_obs : 0;
  const int ns = a.n_sink < npre ? a.n_sink : npre;
  const int i = c * 256 + threadIdx.x;   // candidate index
  const int ncand = npre - ns;
  if (c == 0 && threadIdx.x == 0) {
    a.seg_begin[pair] = (int)(pair * a.max_len);
    a.seg_end[pair] = (int)(pair * a.max_len) + ncand;
  }
  if (i >= ncand) return;
  const int p = ns + i;
  const float* s = a.scores + pair * a.max_len;
  float sum = 0.0f;
#pragma unroll
  for (int d = -3; d <= 3; ++d) {
    const int t = p + d;
    sum += (t >= 0 && t < npre) ? s[t] : 0.0f;
  }
  a.keys[pair * a.max_len + i] = sum * (1.0f / 7.0f);
  a.vals[pair * a.max_len + i] = p;
}

// Forced positions and the first k sorted candidates, ascending, through an
// LDS bitmap of the pair's positions.
__global__ __launch_bounds__(1024) void snap_emit_kernel(SnapArgs a) {
  __shared__ uint32_t bm[kSnapMaxLen / 32];
  __shared__ int wsum[1024 / kWave];
  const int g = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int L = geo.L < a.max_len ? geo.L : a.max_len;
  const int npre = L > a.n_obs ? L - a.n_obs : 0;
  const int ns = a.n_sink < npre ? a.n_sink : npre;
  const int nw = (L + 31) / 32;
  for (int i = tid; i < nw; i += 1024) bm[i] = 0u;
  __syncthreads();
  for (int t = tid; t < L; t += 1024)
    if (t < ns || t >= npre) atomicOr(&bm[t >> 5], 1u << (t & 31));
  const int nforced = ns + (L - npre);
  int k = a.budget - nforced;
  const int ncand = npre - ns;
  k = k < 0 ? 0 : (k > ncand ? ncand : k);
  for (int i = tid; i < k; i += 1024) {
    const int t = a.sorted_vals[pair * a.max_len + i];
    atomicOr(&bm[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  // ascending emission: each thread owns a run of words
  const int wpt = (nw + 1023) / 1024;
  const int w0 = tid * wpt, w1 = w0 + wpt < nw ? w0 + wpt : nw;
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  const int lane = tid & 63, wave = tid >> 6;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < 1024 / kWave; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int pos = before + incl - cnt;
  int32_t* out = a.selected + pair * a.budget;
  for (int w = w0; w < w1; ++w) {
    uint32_t x = bm[w];
    while (x) {
      const int b = __ffs(x) - 1;
      x &= x - 1u;
      if (pos < a.budget) out[pos] = 32 * w + b;
      ++pos;
    }
  }
  const int stot = total < a.budget ? total : a.budget;
  for (int i = stot + tid; i < a.budget; i += 1024) out[i] = -1;
  if (tid == 0) a.counts[pair] = stot;
}

template <int D>
__global__ __launch_bounds__(256) void snap_gather_kernel(SnapArgs a, int budget_pad) {
  // one wave per kept position: D bf16 of K and of V
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), g = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63;
  if (i >= budget_pad) return;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int cnt = a.counts[pair];
  const int t = i < cnt && i < a.budget ? a.selected[pair * a.budget + i] : -1;
  int page = -1;
  if (t >= 0 && t < geo.L && t / 16 < geo.nb) page = a.b.indices[geo.page_base + t / 16];
  if (page >= a.b.num_pages) page = -1;
  constexpr int EPL = D / kWave;   // elements per lane: 1 or 2
  uint16_t* ko = a.k_out + (pair * budget_pad + i) * D + EPL * lane;
  uint16_t* vo = a.v_out + (pair * budget_pad + i) * D + EPL * lane;
  const size_t src = (((size_t)(uint32_t)(page >= 0 ? page : 0) * a.num_kv_heads + g) * 16 +
                      (t >= 0 ? (t & 15) : 0)) * D + EPL * lane;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    ko[e] = page >= 0 ? a.k_pool[src + e] : (uint16_t)0;
    vo[e] = page >= 0 ? a.v_pool[src + e] : (uint16_t)0;
  }
}

size_t snap_sort_bytes(int pairs, int max_len) {
  size_t bytes = 0;
  hipcub::DeviceSegmentedRadixSort::SortPairsDescending(
      nullptr, bytes, (const float*)nullptr, (float*)nullptr, (const int*)nullptr, (int*)nullptr,
      pairs * max_len, pairs, (const int*)nullptr, (const int*)nullptr, 0, 32, (hipStream_t)0);
  return bytes;
}

hipError_t launch_snapkv_select(const SnapArgs& a, hipStream_t st) {
  const int pairs = a.b.batch * a.num_kv_heads;
  const dim3 grid(a.n_chunks, a.num_kv_heads, a.b.batch);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((snap_stats_kernel<128>), grid, dim3(kSnapChunk), 0, st, a);
  else
    hipLaunchKernelGGL((snap_stats_kernel<64>), grid, dim3(kSnapChunk), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(snap_rowstat_kernel, dim3(pairs), dim3(kSnapRows), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.head_dim == 128)
    hipLaunchKernelGGL((snap_score_kernel<128>), grid, dim3(kSnapChunk), 0, st, a);
  else
    hipLaunchKernelGGL((snap_score_kernel<64>), grid, dim3(kSnapChunk), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(snap_pool_kernel, dim3((a.max_len + 255) / 256, a.num_kv_heads, a.b.batch),
                     dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  size_t bytes = a.sort_bytes;
  e = hipcub::DeviceSegmentedRadixSort::SortPairsDescending(
      a.sort_tmp, bytes, a.keys, a.sorted_keys, a.vals, a.sorted_vals, pairs * a.max_len, pairs,
      a.seg_begin, a.seg_end, 0, 32, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(snap_emit_kernel, dim3(a.num_kv_heads, a.b.batch), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_snapkv_gather(const SnapArgs& a, int budget_pad, hipStream_t st) {
  const dim3 grid((budget_pad + 3) / 4, a.num_kv_heads, a.b.batch);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((snap_gather_kernel<128>), grid, dim3(256), 0, st, a, budget_pad);
  else
    hipLaunchKernelGGL((snap_gather_kernel<64>), grid, dim3(256), 0, st, a, budget_pad);
  return hipGetLastError();
}

}  // namespace ls

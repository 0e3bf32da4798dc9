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
// Kernels (per (request, KV head) pair):
//   snap_stats_kernel   per chunk of 256 positions and query row: max and sum
//                       of exp of the logits (the logits of a 16-row x
//                       16-position tile are one bf16 MFMA chain, D / 32
//                       16x16x32 steps; each wave takes 64 positions);
//   snap_rowstat_kernel per row: the max and 1 / sum over all chunks;
//   snap_score_kernel   per position: sum over rows of exp(z - max) / sum,
//                       the same MFMA tiles (rows summed in a fixed order:
//                       deterministic);
//   snap_pool_kernel    the width-7 average of the candidates;
//   snap_select_kernel  one workgroup: exact radix select of the candidates
//                       by the order-preserving key of the averaged score
//                       (four 8-bit digits from the top; the last digit's
//                       bucket holds the threshold key, whose candidates are
//                       taken lowest position first), the forced positions,
//                       and the ascending emission from an LDS bitmap;
//   snap_gather_kernel  K and V rows of the kept positions, contiguous.
// This runs once per prompt, not per decode step.
#include "dev_mfma.h"
#include "ls_internal.h"

namespace ls {

constexpr int kSnapChunk = 256;   // positions per workgroup (4 waves x 64)
constexpr int kSnapRows = kSnapMaxObs * 4;
constexpr int kSnapSelThreads = 1024;

// The pair's W x 4 query rows (row w * 4 + h, head g * 4 + h) into LDS,
// rows padded by 8 elements (the MFMA operand reads of 16 rows then hit
// distinct banks).
template <int D>
constexpr int snap_qstride() { return D + 8; }

template <int D>
__device__ __forceinline__ void snap_load_q(const SnapArgs& a, int r, int g, uint16_t* q_lds) {
  const int rows = a.n_obs * 4;
  for (int i = threadIdx.x; i < rows * D / 8; i += kSnapChunk) {
    const int row = i / (D / 8), c = i % (D / 8);
    const int w = row / 4, h = row % 4;
    const uint4 v = *reinterpret_cast<const uint4*>(
        a.q_obs + (((size_t)r * a.n_obs + w) * a.num_q_heads + g * 4 + h) * D + 8 * c);
    *reinterpret_cast<uint4*>(q_lds + (size_t)row * snap_qstride<D>() + 8 * c) = v;
  }
}

// This wave's 64 positions as 4 MFMA B operands (16 positions each): lane i
// holds dims 32 j + 8 (i / 16) .. + 8 of position t * 16 + i % 16. Returns
// the bit mask of tiles whose position of this lane is a valid cache token.
template <int D>
__device__ __forceinline__ unsigned snap_load_k(const SnapArgs& a, int g, const ReqGeom& geo,
                                                int p0, int Lc, uint4 (&kb)[4][D / 32]) {
  const int lane = threadIdx.x & 63;
  unsigned okm = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int p = p0 + t * 16 + (lane & 15);
    const int blk = p / 16;
    int page = p < Lc && blk < geo.nb ? a.b.indices[geo.page_base + blk] : -1;
    if (page < 0 || page >= a.b.num_pages) page = -1;
    okm |= (unsigned)(page >= 0) << t;
    const uint16_t* kr = a.k_pool + (((size_t)(uint32_t)(page >= 0 ? page : 0) * a.num_kv_heads + g) * 16 +
                                     (p & 15)) * D + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
      kb[t][j] = page >= 0 ? *reinterpret_cast<const uint4*>(kr + 32 * j) : make_uint4(0, 0, 0, 0);
  }
  return okm;
}

// Logits of rows rt * 16 .. + 16 against position tile t: lane i gets rows
// rt * 16 + 4 (i / 16) + jj (query w = rt * 4 + i / 16, head jj) of position
// t * 16 + i % 16, unscaled.
template <int D>
__device__ __forceinline__ f32x4_t snap_logits(const uint16_t* q_lds, int rt, const uint4* kb) {
  const int lane = threadIdx.x & 63;
  const uint16_t* qr = q_lds + (size_t)(rt * 16 + (lane & 15)) * snap_qstride<D>() + 8 * (lane >> 4);
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    acc = mfma_16x16x32(*reinterpret_cast<const uint4*>(qr + 32 * j), kb[j], acc);
  return acc;
}

// (m, s) <- the merge of two (max, sum of exp2(z - max)) states.
__device__ __forceinline__ void snap_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -__builtin_huge_valf()) return;
  s = s * exp2f(m - mn) + s2 * exp2f(m2 - mn);
  m = mn;
}

template <int D>
__global__ __launch_bounds__(kSnapChunk) void snap_stats_kernel(SnapArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kSnapRows * snap_qstride<D>()];
  __shared__ float red_m[kSnapChunk / kWave][kSnapRows], red_s[kSnapChunk / kWave][kSnapRows];
  const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const int Lc = geo.L < a.max_len ? geo.L : a.max_len;   // positions past max_len are not read
  const int p0 = c * kSnapChunk + wave * 64;
  snap_load_q<D>(a, r, g, q_lds);
  uint4 kb[4][D / 32];
  const unsigned okm = snap_load_k<D>(a, g, geo, p0, Lc, kb);
  __syncthreads();
  const int rows = a.n_obs * 4;
  for (int rt = 0; rt < (rows + 15) / 16; ++rt) {
    const int w = rt * 4 + (lane >> 4);
    // this lane's logits (4 rows x 4 positions), masked; then per row the
    // maximum over the row group's 64 positions and the sum of exp2(z - max)
    float z[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4_t zt = snap_logits<D>(q_lds, rt, kb[t]);
      const int p = p0 + t * 16 + (lane & 15);
      const bool ok = ((okm >> t) & 1u) && w < a.n_obs && p <= Lc - a.n_obs + w;   // causal
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) z[t][jj] = ok ? zt[jj] * a.sm_scale_log2 : -__builtin_huge_valf();
    }
    float m[4], s[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      m[jj] = fmaxf(fmaxf(z[0][jj], z[1][jj]), fmaxf(z[2][jj], z[3][jj]));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) m[jj] = fmaxf(m[jj], __shfl_xor(m[jj], off, kWave));
      s[jj] = 0.0f;
      if (m[jj] != -__builtin_huge_valf()) {
#pragma unroll
        for (int t = 0; t < 4; ++t) s[jj] += exp2f(z[t][jj] - m[jj]);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) s[jj] += __shfl_xor(s[jj], off, kWave);
    }
    if ((lane & 15) == 0 && w < a.n_obs) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        red_m[wave][w * 4 + jj] = m[jj];
        red_s[wave][w * 4 + jj] = s[jj];
      }
    }
  }
  __syncthreads();
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  for (int row = tid; row < rows; row += kSnapChunk) {
    float m = -__builtin_huge_valf(), sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kSnapChunk / kWave; ++w) snap_merge(m, sum, red_m[w][row], red_s[w][row]);
    float* st = a.stats + ((pair * a.n_chunks + c) * kSnapRows + row) * 2;
    st[0] = m;
    st[1] = sum;
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
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kSnapRows * snap_qstride<D>()];
  __shared__ float rm[kSnapRows], rinv[kSnapRows];
  const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int Lc = geo.L < a.max_len ? geo.L : a.max_len;
  const int p0 = c * kSnapChunk + wave * 64;
  snap_load_q<D>(a, r, g, q_lds);
  uint4 kb[4][D / 32];
  const unsigned okm = snap_load_k<D>(a, g, geo, p0, Lc, kb);
  const int rows = a.n_obs * 4;
  for (int row = tid; row < rows; row += kSnapChunk) {
    rm[row] = a.rowstat[(pair * kSnapRows + row) * 2];
    rinv[row] = a.rowstat[(pair * kSnapRows + row) * 2 + 1];
  }
  __syncthreads();
  float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // this lane's position of each tile, its 4 rows
  for (int rt = 0; rt < (rows + 15) / 16; ++rt) {
    const int w = rt * 4 + (lane >> 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4_t z = snap_logits<D>(q_lds, rt, kb[t]);
      const int p = p0 + t * 16 + (lane & 15);
      const bool ok = ((okm >> t) & 1u) && w < a.n_obs && p <= Lc - a.n_obs + w;
      if (ok) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          sc[t] += exp2f(z[jj] * a.sm_scale_log2 - rm[w * 4 + jj]) * rinv[w * 4 + jj];
      }
    }
  }
  // sum over the 4 row groups (lanes i, i ^ 16, i ^ 32, i ^ 48), fixed order
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sc[t] += __shfl_xor(sc[t], 16, kWave);
    sc[t] += __shfl_xor(sc[t], 32, kWave);
  }
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p = p0 + t * 16 + lane;
      if (p < a.max_len) a.scores[pair * a.max_len + p] = p < Lc ? sc[t] : 0.0f;
    }
  }
}

// Averaged scores of the candidates [n_sink, L - W): candidate i (position
// n_sink + i) at keys[pair * max_len + i].
__global__ __launch_bounds__(256) void snap_pool_kernel(SnapArgs a) {
  const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int Lc = geo.L < a.max_len ? geo.L : a.max_len;
  const int npre = Lc > a.n_obs ? Lc - a.n_obs : 0;
  const int ns = a.n_sink < npre ? a.n_sink : npre;
  const int i = c * 256 + threadIdx.x;   // candidate index
  const int ncand = npre - ns;
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
}

// Exclusive prefix sum of v over the workgroup (NT threads) in thread
// order, and the total. One barrier; wsum has NT / 64 entries.
template <int NT>
__device__ __forceinline__ int snap_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    before += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  *total = tot;
  return before + incl - v;
}

// The selection of one pair: forced positions, the k best candidates by
// (averaged score descending, position ascending), ascending output.
__global__ __launch_bounds__(kSnapSelThreads) void snap_select_kernel(SnapArgs a) {
  constexpr int NT = kSnapSelThreads;
  __shared__ uint32_t bm[kSnapMaxLen / 32];
  __shared__ int hist[256];
  __shared__ int wsum[2][NT / kWave];
  __shared__ int bsel[3];   // the digit's bucket, candidates above it, candidates in it
  const int g = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int L = geo.L < a.max_len ? geo.L : a.max_len;
  const int npre = L > a.n_obs ? L - a.n_obs : 0;
  const int ns = a.n_sink < npre ? a.n_sink : npre;
  const int nw = (L + 31) / 32;
  const float* keys = a.keys + pair * a.max_len;
  for (int i = tid; i < nw; i += NT) bm[i] = 0u;
  __syncthreads();
  for (int t = tid; t < L; t += NT)
    if (t < ns || t >= npre) atomicOr(&bm[t >> 5], 1u << (t & 31));
  const int nforced = ns + (L - npre);
  const int ncand = npre - ns;
  int k = a.budget - nforced;
  k = k < 0 ? 0 : (k > ncand ? ncand : k);
  if (k == ncand) {
    for (int i = tid; i < ncand; i += NT) atomicOr(&bm[(ns + i) >> 5], 1u << ((ns + i) & 31));
  } else if (k > 0) {
    // radix select of the k-th largest key, 8 bits at a time from the top
    uint32_t prefix = 0;
    int need = k, neq = 0;
    for (int d = 0; d < 4; ++d) {
      const int shift = 24 - 8 * d;
      for (int i = tid; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < ncand; i += NT) {
        const uint32_t u = score_key(keys[i]);
        if (d == 0 || (u >> (shift + 8)) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid < kWave) {
        // the highest bucket b whose suffix count (candidates in buckets >= b) is >= need
        const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                  h3 = hist[4 * lane + 3];
        const int lsum = h0 + h1 + h2 + h3;
        int incl = lsum;   // suffix over lanes: sum of lanes >= this one
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int u = __shfl_down(incl, off, kWave);
          if (lane + off < 64) incl += u;
        }
        const int s0 = incl, s1 = s0 - h0, s2 = s1 - h1, s3 = s2 - h2;
        int best = -1, above = 0, in = 0;
        if (s0 >= need) { best = 4 * lane; above = s1; in = h0; }
        if (s1 >= need) { best = 4 * lane + 1; above = s2; in = h1; }
        if (s2 >= need) { best = 4 * lane + 2; above = s3; in = h2; }
        if (s3 >= need) { best = 4 * lane + 3; above = s3 - h3; in = h3; }
        const unsigned long long m = __ballot(best >= 0);
        const int hl = 63 - __builtin_clzll(m);
        if (lane == hl) {
          bsel[0] = best;
          bsel[1] = above;
          bsel[2] = in;
        }
      }
      __syncthreads();
      prefix = (prefix << 8) | (uint32_t)bsel[0];
      need -= bsel[1];
      neq = bsel[2];
      __syncthreads();   // bsel and hist are rewritten by the next digit
    }
    // keys above the threshold, and `need` of those equal to it, lowest
    // position first (all of them when need == neq)
    int base = 0;
    for (int i0 = 0; i0 < ncand; i0 += NT) {
      const int i = i0 + tid;
      const uint32_t u = i < ncand ? score_key(keys[i]) : 0u;
      const bool eq = i < ncand && u == prefix;
      bool take = i < ncand && u > prefix;
      if (need == neq) {
        take = take || eq;
      } else {
        int tot;
        const int rank = base + snap_scan<NT>(eq ? 1 : 0, wsum[(i0 / NT) & 1], &tot);
        take = take || (eq && rank < need);
        base += tot;
      }
      if (take) atomicOr(&bm[(ns + i) >> 5], 1u << ((ns + i) & 31));
    }
  }
  __syncthreads();
  // ascending emission: each thread owns a run of words
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = tid * wpt, w1 = w0 + wpt < nw ? w0 + wpt : nw;
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  int total;
  int pos = snap_scan<NT>(cnt, wsum[0], &total);
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
  for (int i = stot + tid; i < a.budget; i += NT) out[i] = -1;
  if (tid == 0) a.counts[pair] = stot;
}

// Kept rows into the contiguous buffers: each lane moves 16 bytes of K and of
// V; a 256-thread workgroup covers 256 * 8 / D positions.
template <int D>
__global__ __launch_bounds__(256) void snap_gather_kernel(SnapArgs a, int budget_pad) {
  constexpr int LPP = D / 8;            // lanes per position (16 or 8)
  constexpr int PPW = 256 / LPP;        // positions per workgroup
  const int g = blockIdx.y, r = blockIdx.z;
  const int i = blockIdx.x * PPW + threadIdx.x / LPP, c = threadIdx.x % LPP;
  if (i >= budget_pad) return;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  const size_t pair = (size_t)r * a.num_kv_heads + g;
  const int cnt = a.counts[pair];
  const int t = i < cnt && i < a.budget ? a.selected[pair * a.budget + i] : -1;
  int page = -1;
  if (t >= 0 && t < geo.L && t / 16 < geo.nb) page = a.b.indices[geo.page_base + t / 16];
  if (page >= a.b.num_pages) page = -1;
  const size_t src = (((size_t)(uint32_t)(page >= 0 ? page : 0) * a.num_kv_heads + g) * 16 +
                      (t >= 0 ? (t & 15) : 0)) * D + 8 * c;
  const uint4 kv = page >= 0 ? *reinterpret_cast<const uint4*>(a.k_pool + src) : make_uint4(0, 0, 0, 0);
  const uint4 vv = page >= 0 ? *reinterpret_cast<const uint4*>(a.v_pool + src) : make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint4*>(a.k_out + (pair * budget_pad + i) * D + 8 * c) = kv;
  *reinterpret_cast<uint4*>(a.v_out + (pair * budget_pad + i) * D + 8 * c) = vv;
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
  hipLaunchKernelGGL(snap_select_kernel, dim3(a.num_kv_heads, a.b.batch), dim3(kSnapSelThreads), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_snapkv_gather(const SnapArgs& a, int budget_pad, hipStream_t st) {
  const int ppw = 256 / (a.head_dim / 8);
  const dim3 grid((budget_pad + ppw - 1) / ppw, a.num_kv_heads, a.b.batch);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((snap_gather_kernel<128>), grid, dim3(256), 0, st, a, budget_pad);
  else
    hipLaunchKernelGGL((snap_gather_kernel<64>), grid, dim3(256), 0, st, a, budget_pad);
  return hipGetLastError();
}

}  // namespace ls

// PQ32 codes of indexer keys and coarse scoring from them (LeanSparse §5,
// "Approximate scoring with PQ", Eq. 6).
//
// A 128-dim indexer key x = scale * fp8 is cut into 32 subvectors of 4 dims;
// each is stored as the one-byte index of its nearest centroid in that
// subspace's codebook of 256 bf16 centroids ([32][256][4] bf16, 64 KB).
//
// Encoding decides an integer from floating point, so the distance is fixed
// to the bit: float64, d_t = x_t - c_t, ((d0 d0 + d1 d1) + d2 d2) + d3 d3 with
// every operation rounded once (no contraction), ties to the lowest centroid.
// x_t is exact in float64 (a 24-bit scale times a 4-bit fp8 value).
//
// Codebook training is Lloyd's k-means with order-independent means: each
// member value v is added as the integer rint(v * 2^24) with 64-bit integer
// atomics (first within the workgroup in LDS, then into global sums), so the
// sums, and the means (sum / count) * 2^-24 rounded once to bf16, do not
// depend on the order of the additions.
//
// Coarse scoring reads 32 bytes of codes per token instead of 128 + 4 bytes
// of fp8 key and scale. The 64 KB codebook sits in LDS; a lane rebuilds its
// slice of the MFMA B operand (key^T) from 8 code bytes: k-step s of lane
// group kq covers dims 32 kq + 8 s .. + 8, i.e. subspaces 8 kq + 2 s and
// 8 kq + 2 s + 1, one 8-byte LDS read each. The rest (weighted ReLU over the
// heads, score range, histogram, mark + finish) is the token top-k of the
// learned indexer.
#include "dev_indexer.h"
#include "dev_mfma.h"

namespace ls {

// Key token i of the listed pages: its row (page * P + slot), or -1.
__device__ __forceinline__ long long pq_key_row(const PqArgs& a, long long i) {
  const int P = a.page_size;
  if (i < 0 || i >= (long long)a.n_pages * P) return -1;
  const int page = a.page_ids[i / P];
  if (page < 0 || page >= a.num_pages) return -1;
  return (long long)page * P + (int)(i % P);
}

// Subvector j of key row `row`, exact in float64.
__device__ __forceinline__ void pq_subvector(const PqArgs& a, long long row, int j, double x[4]) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(a.keys + row * 128 + 4 * j);
  const double sc = a.scales ? (double)a.scales[row] : 1.0;
  const uint32_t lo = fp8x2_to_bf16x2(w, false), hi = fp8x2_to_bf16x2(w, true);
  x[0] = sc * (double)__uint_as_float(lo << 16);
  x[1] = sc * (double)__uint_as_float(lo & 0xffff0000u);
  x[2] = sc * (double)__uint_as_float(hi << 16);
  x[3] = sc * (double)__uint_as_float(hi & 0xffff0000u);
}

// Nearest centroid of x among cb[0..255] (float64 rows in LDS).
__device__ __forceinline__ int pq_nearest(const double x[4], const double (*cb)[4]) {
#pragma clang fp contract(off)
  double best = __builtin_huge_val();
  int arg = 0;
  for (int c = 0; c < kPqCent; ++c) {
    const double d0 = x[0] - cb[c][0], d1 = x[1] - cb[c][1];
    const double d2 = x[2] - cb[c][2], d3 = x[3] - cb[c][3];
    const double dist = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
    if (dist < best) {
      best = dist;
      arg = c;
    }
  }
  return arg;
}

// One thread per listed token, one subspace per grid row: the code, and
// (training) the fixed-point sums and counts of the chosen centroids.
__global__ __launch_bounds__(256) void pq_assign_kernel(PqArgs a) {
  __shared__ double cb[kPqCent][4];
  __shared__ unsigned long long s_sum[kPqCent][4];
  __shared__ uint32_t s_cnt[kPqCent];
  const int j = blockIdx.y, tid = threadIdx.x;
  {
    const uint2 c = *reinterpret_cast<const uint2*>(a.codebooks + ((size_t)j * kPqCent + tid) * 4);
    cb[tid][0] = (double)__uint_as_float(c.x << 16);
    cb[tid][1] = (double)__uint_as_float(c.x & 0xffff0000u);
    cb[tid][2] = (double)__uint_as_float(c.y << 16);
    cb[tid][3] = (double)__uint_as_float(c.y & 0xffff0000u);
    if (a.sums) {
      s_sum[tid][0] = s_sum[tid][1] = s_sum[tid][2] = s_sum[tid][3] = 0ull;
      s_cnt[tid] = 0u;
    }
  }
  __syncthreads();
  const long long i = (long long)blockIdx.x * 256 + tid;
  const long long row = pq_key_row(a, i);
  if (row >= 0) {
    double x[4];
    pq_subvector(a, row, j, x);
    const int c = pq_nearest(x, cb);
    if (a.codes) a.codes[row * kPqSub + j] = (uint8_t)c;
    if (a.sums) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const long long v = (long long)rint(x[t] * (double)(1 << kPqFixedBits));
        atomicAdd(&s_sum[c][t], (unsigned long long)v);   // two's complement: a signed sum
      }
      atomicAdd(&s_cnt[c], 1u);
    }
  }
  if (a.sums) {
    __syncthreads();
    const uint32_t n = s_cnt[tid];
    if (n) {
      atomicAdd(a.counts + (size_t)j * kPqCent + tid, n);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        atomicAdd(a.sums + ((size_t)j * kPqCent + tid) * 4 + t, s_sum[tid][t]);
    }
  }
}

// Centroid c of subspace j = subvector j of listed token init[c], rounded
// to bf16 (zero for an init token outside the listed pages); sums and
// counts cleared.
__global__ __launch_bounds__(256) void pq_init_kernel(PqArgs a, const int32_t* init) {
  const int j = blockIdx.x, c = threadIdx.x;
  const long long row = pq_key_row(a, init[c]);
  double x[4] = {0.0, 0.0, 0.0, 0.0};
  if (row >= 0) pq_subvector(a, row, j, x);
  uint16_t* o = a.codebooks + ((size_t)j * kPqCent + c) * 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    o[t] = f64_to_bf16_rne(x[t]);
    a.sums[((size_t)j * kPqCent + c) * 4 + t] = 0ull;
  }
  a.counts[(size_t)j * kPqCent + c] = 0u;
}

// Centroids with members become their fixed-point mean; sums and counts are
// cleared for the next iteration.
__global__ __launch_bounds__(256) void pq_update_kernel(PqArgs a) {
  const int j = blockIdx.x, c = threadIdx.x;
  const size_t e = (size_t)j * kPqCent + c;
  const uint32_t n = a.counts[e];
  if (n) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const long long s = (long long)a.sums[e * 4 + t];
      const double m = ((double)s / (double)n) * (1.0 / (double)(1 << kPqFixedBits));
      a.codebooks[e * 4 + t] = f64_to_bf16_rne(m);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) a.sums[e * 4 + t] = 0ull;
  a.counts[e] = 0u;
}

// Encoding of a few pages (the ones that filled at a step): the 256
// centroids of subspace j are spread over a wave's lanes (4 each, in
// registers), so a code costs 4 distances per lane and a wave reduction of
// (distance, index) that keeps the lowest index among equal distances (the
// same result as the serial scan). Each wave codes kPqEncTokens tokens, their
// key loads issued before the first distance.
constexpr int kPqEncTokens = 4;

__global__ __launch_bounds__(256) void pq_encode_kernel(PqArgs a) {
#pragma clang fp contract(off)
  const int j = blockIdx.y, lane = threadIdx.x & 63;
  const long long t0 = ((long long)blockIdx.x * 4 + wave_id()) * kPqEncTokens;
  long long row[kPqEncTokens];
#pragma unroll
  for (int t = 0; t < kPqEncTokens; ++t) row[t] = pq_key_row(a, t0 + t);
  double x[kPqEncTokens][4];
#pragma unroll
  for (int t = 0; t < kPqEncTokens; ++t) pq_subvector(a, row[t] >= 0 ? row[t] : 0, j, x[t]);
  double c[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint2 v = *reinterpret_cast<const uint2*>(a.codebooks +
                                                    ((size_t)j * kPqCent + lane + 64 * m) * 4);
    c[m][0] = (double)__uint_as_float(v.x << 16);
    c[m][1] = (double)__uint_as_float(v.x & 0xffff0000u);
    c[m][2] = (double)__uint_as_float(v.y << 16);
    c[m][3] = (double)__uint_as_float(v.y & 0xffff0000u);
  }
#pragma unroll
  for (int t = 0; t < kPqEncTokens; ++t) {
    double best = __builtin_huge_val();
    int arg = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {   // ascending centroid index: strict < keeps the lowest
      const double d0 = x[t][0] - c[m][0], d1 = x[t][1] - c[m][1];
      const double d2 = x[t][2] - c[m][2], d3 = x[t][3] - c[m][3];
      const double dist = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
      if (dist < best) {
        best = dist;
        arg = lane + 64 * m;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int oa = __shfl_xor(arg, off);
      if (ob < best || (ob == best && oa < arg)) {
        best = ob;
        arg = oa;
      }
    }
    if (lane == 0 && row[t] >= 0) a.codes[row[t] * kPqSub + j] = (uint8_t)arg;
  }
}

hipError_t launch_pq_encode(const PqArgs& a, hipStream_t st) {
  const long long n = (long long)a.n_pages * a.page_size;
  const long long per_block = 4 * kPqEncTokens;
  hipLaunchKernelGGL(pq_encode_kernel, dim3((unsigned)((n + per_block - 1) / per_block), kPqSub),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pq_train(const PqArgs& a, const int32_t* init_tokens, int iters,
                           hipStream_t st) {
  const long long n = (long long)a.n_pages * a.page_size;
  hipLaunchKernelGGL(pq_init_kernel, dim3(kPqSub), dim3(kPqCent), 0, st, a, init_tokens);
  hipError_t e = hipGetLastError();
  PqArgs t = a;
  t.codes = nullptr;
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    hipLaunchKernelGGL(pq_assign_kernel, dim3((unsigned)((n + 255) / 256), kPqSub), dim3(256),
                       0, st, t);
    e = hipGetLastError();
    if (e != hipSuccess) break;
    hipLaunchKernelGGL(pq_update_kernel, dim3(kPqSub), dim3(kPqCent), 0, st, t);
    e = hipGetLastError();
  }
  return e;
}

// ------------------------------------------------------- coarse scoring ----

constexpr int kPqPrefetch = 4;   // code tiles in flight per wave (8 bytes per lane each)

template <int NHT>
struct PqScoreLds {
  union {
    uint4 q[NHT][4][kWave];            // the q operand, staged once
    uint2 cb[kPqSub * kPqCent];        // the codebook (4 bf16 per centroid)
  } u;
  float red[2 * kIdxWaves];
  int pg[kIdxMaxTilesPerWg + 1];       // page ids of the workgroup's blocks
};

template <int NHT>
__global__ __launch_bounds__(kIdxThreads, 2) void pq_score_kernel(IndexerArgs a) {
  constexpr int NS = kPqPrefetch, H = 16 * NHT;
  __shared__ PqScoreLds<NHT> sh;
  const int r = blockIdx.y, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int P = a.b.page_size, PS = __builtin_ctz((unsigned)P);
  const int upw = a.tiles_per_wg * 16;
  const int u0 = blockIdx.x * upw;
  const IdxUnits gu = idx_units(a, r);   // the complete pages' tokens
  if (blockIdx.x == 0) idx_clear_request<kIdxThreads>(a, r);
  if (u0 >= gu.n) return;

  const int bi0 = u0 >> PS;
  const int npg = (upw + P - 1) >> PS;
  for (int i = tid; i < npg; i += kIdxThreads) {
    const int blk = bi0 + i;
    int page = -1;
    if (blk < gu.nb) {
      const int p = a.b.indices[gu.page_base + blk];
      page = (p >= 0 && p < a.b.num_pages) ? p : -2;   // -2: bad page id, scores 0
    }
    sh.pg[i] = page;
  }

  // q as the A operand (rows = heads 16 ht + col, k-step s of lane group kq
  // = dims 32 kq + 8 s .. + 8), through LDS into registers
  float wv[NHT][4];
  {
    constexpr int NQ = NHT * 4 * kWave / kIdxThreads;
    uint4 qv[NQ];
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int e = tid + m * kIdxThreads;
      const int ht = e / (4 * kWave), s = (e / kWave) % 4, ln = e % kWave;
      qv[m] = ldg16(a.q + ((size_t)r * H + 16 * ht + (ln & 15)) * kIdxDim + 32 * (ln >> 4) + 8 * s);
    }
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int e = tid + m * kIdxThreads;
      sh.u.q[e / (4 * kWave)][(e / kWave) % 4][e % kWave] = qv[m];
    }
  }
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)r * H + 16 * ht + 4 * kq + i];
  __syncthreads();
  uint4 qr[NHT][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) qr[ht][s2] = sh.u.q[ht][s2][lane];
  __syncthreads();
  {
    // the codebook: 4,096 16-byte pieces, every load of a thread issued first
    constexpr int NC = kPqSub * kPqCent * 8 / 16 / kIdxThreads;
    const uint4* src = reinterpret_cast<const uint4*>(a.codebooks);
    uint4 cv[NC];
#pragma unroll
    for (int m = 0; m < NC; ++m) cv[m] = ldg16(src + tid + m * kIdxThreads);
    uint4* dst = reinterpret_cast<uint4*>(sh.u.cb);
#pragma unroll
    for (int m = 0; m < NC; ++m) dst[tid + m * kIdxThreads] = cv[m];
  }
  __syncthreads();

  const int ntw = a.tiles_per_wg / kIdxWaves;
  float* srow = a.scores + (size_t)r * a.max_units + u0;
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.keys);
  auto issue = [&](int k, uint2& d, bool& bad) {
    const int u = u0 + 16 * (wave + kIdxWaves * k) + col;
    const int page = k < ntw ? sh.pg[(u >> PS) - bi0] : -1;
    bad = page == -2;
    const size_t row = (size_t)(uint32_t)(page >= 0 ? page : 0) * P + (u & (P - 1));
    d = *reinterpret_cast<const uint2*>(codes + row * kPqSub + 8 * kq);
  };
  uint2 buf[NS];
  bool bad[NS];
  float rmn = __builtin_inff(), rmx = -__builtin_inff();   // range of this thread's valid scores
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    issue(s, buf[s], bad[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int k0 = 0; k0 < ntw; k0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int k = k0 + s;
      const uint2 c = buf[s];
      const bool bd = bad[s];
      __builtin_amdgcn_sched_barrier(0);
      issue(k + NS, buf[s], bad[s]);
      __builtin_amdgcn_sched_barrier(0);
      if (k < ntw) {
        uint4 kb[4];
        const uint32_t cw[2] = {c.x, c.y};
        const int jb = 8 * kq;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const uint32_t w = cw[s2 >> 1] >> (16 * (s2 & 1));
          const uint2 e0 = sh.u.cb[(jb + 2 * s2) * kPqCent + (w & 0xffu)];
          const uint2 e1 = sh.u.cb[(jb + 2 * s2 + 1) * kPqCent + ((w >> 8) & 0xffu)];
          kb[s2] = bd ? make_uint4(0, 0, 0, 0) : make_uint4(e0.x, e0.y, e1.x, e1.y);
        }
        // k-step outer, head tile inner: independent products back to back
        f32x4_t acc[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) acc[ht] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) acc[ht] = mfma_16x16x32(qr[ht][s2], kb[s2], acc[ht]);
        float v = 0.0f;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) v = fmaf(wv[ht][i], relu_bits(acc[ht][i]), v);
        v = xor_pair_sum<16>(v);
        v = xor_pair_sum<32>(v);
        v += 0.0f;   // -0 -> +0: equal scores get equal keys
        if (kq == 0) {
          const int ul = 16 * (wave + kIdxWaves * k) + col;
          // every token of a complete page is a unit (no memory read here:
          // its wait would also wait for the code tiles in flight)
          const bool valid = u0 + ul < gu.n;
          if (valid) {
            rmn = fminf(rmn, v);
            rmx = fmaxf(rmx, v);
          }
          if (u0 + ul < gu.n) srow[ul] = valid ? v : 0.0f;
        }
      }
    }
  }
  idx_range_reduce<kIdxThreads>(rmn, rmx, sh.red);
  if (tid == 0)
    a.range[(size_t)r * (a.max_units / kIdxMinWgUnits) + blockIdx.x] = make_float2(rmn, rmx);
}

hipError_t launch_pq_select(const IndexerArgs& a, hipStream_t st) {
  const int upw = a.tiles_per_wg * 16;
  dim3 grid((a.max_units + upw - 1) / upw, a.b.batch);
  switch (a.num_heads) {
    case 16: hipLaunchKernelGGL((pq_score_kernel<1>), grid, dim3(kIdxThreads), 0, st, a); break;
    case 32: hipLaunchKernelGGL((pq_score_kernel<2>), grid, dim3(kIdxThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((pq_score_kernel<4>), grid, dim3(kIdxThreads), 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_indexer_hist(a, st);
  if (e != hipSuccess) return e;
  return launch_indexer_mark(a, st);
}

// --------------------------------------------------------- miss filter ----

// LeanSparse §5, "Retrieving and refining candidates": before the original
// keys of the candidates are fetched, every candidate whose key is resident
// is kept, and a miss is kept only when its approximate score is at least
// theta = s_(j) - sd, j = min(k, n), s_(j) the j-th largest approximate score
// of the n candidates and sd their sample standard deviation (0 for n < 2),
// both in float64. One workgroup per request
// (consecutive entries, so that the kept ones compact in order): float64
// sums reduced in a fixed order (the result does not depend on scheduling),
// the j-th largest by a radix select over the order-preserving score key
// (four 8-bit digits), then a workgroup scan places the kept candidates.
// Eight candidates per thread.
constexpr int kPqFilterThreads = 512;
constexpr int kPqFilterPer = kPqFilterMaxCand / kPqFilterThreads;
constexpr int kPqFilterWaves = kPqFilterThreads / kWave;

struct PqFilterLds {
  double dred[2][kPqFilterWaves];
  int ired[kPqFilterWaves];
  uint32_t hist[2][256];   // the radix rounds alternate between two histograms
  uint32_t kmin[kPqFilterWaves], kmax[kPqFilterWaves];
  int digit[2], above[2];
};

// Workgroup sums (float64) of a and b in a fixed order: lanes by a
// butterfly, then the waves in order. Every thread gets them. Synchronises.
__device__ __forceinline__ void pq_block_sum2(double& a, double& b, double (*red)[kPqFilterWaves]) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    a += __shfl_xor(a, o, kWave);
    b += __shfl_xor(b, o, kWave);
  }
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[0][wave] = a;
    red[1][wave] = b;
  }
  __syncthreads();
  a = 0.0;
  b = 0.0;
#pragma unroll
  for (int w = 0; w < kPqFilterWaves; ++w) {
    a += red[0][w];
    b += red[1][w];
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup in thread order; *total = sum.
__device__ __forceinline__ int pq_block_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int inc = wave_incl_scan(v, lane);
  if (lane == kWave - 1) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPqFilterWaves; ++w) {
    before += w < wave ? red[w] : 0;
    tot += red[w];
  }
  *total = tot;
  return before + inc - v;
}

// The float whose score_key is k.
__device__ __forceinline__ float pq_key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(kPqFilterThreads) void pq_filter_kernel(PqFilterArgs a) {
  __shared__ PqFilterLds sh;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
  int c = a.counts[r];
  c = c < 0 ? 0 : (c > a.cap ? a.cap : c);
  // this thread's candidates (entries kPqFilterPer tid + j), every load of a
  // round issued before the dependent ones
  int tok[kPqFilterPer];
  float sc[kPqFilterPer];
  bool val[kPqFilterPer], res[kPqFilterPer];
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j) {
    const int i = kPqFilterPer * tid + j;
    tok[j] = i < c ? a.candidates[(size_t)r * a.cap + i] : -1;
  }
  uint32_t rw[kPqFilterPer];
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j) {
    val[j] = tok[j] >= 0 && tok[j] < a.score_stride;   // other ids are not candidates
    sc[j] = val[j] ? a.scores[(size_t)r * a.score_stride + tok[j]] : 0.0f;
    const int w = tok[j] >> 5;
    rw[j] = (val[j] && w < a.resident_words) ? a.resident[(size_t)r * a.resident_words + w] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j) res[j] = (rw[j] >> (tok[j] & 31)) & 1u;
  if (tid < 256) sh.hist[0][tid] = 0u;
  // n and the mean, then the sample standard deviation
  double nsum = 0.0, s1 = 0.0;
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j) {
    nsum += val[j] ? 1.0 : 0.0;
    s1 += val[j] ? (double)sc[j] : 0.0;
  }
  pq_block_sum2(nsum, s1, sh.dred);
  const int n = (int)nsum;
  const double mean = s1 / (double)(n > 0 ? n : 1);
  double s2 = 0.0, unused = 0.0;
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j) {
    const double d = (double)sc[j] - mean;
    s2 += val[j] ? d * d : 0.0;
  }
  pq_block_sum2(s2, unused, sh.dred);
  const double sd = n >= 2 ? sqrt(s2 / (double)(n - 1)) : 0.0;
  // the j-th largest score, j = min(k, n): radix select over the keys in
  // 8-bit digits below the bits that every key shares (the top bits of
  // scores of one magnitude agree, and counting them would pile every
  // candidate onto one LDS counter); round d counts into hist[d & 1] while
  // the other one is cleared for the next round
  double theta = 0.0;
  if (n > 0) {
    int need = a.topk < n ? a.topk : n;
    uint32_t key[kPqFilterPer], kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kPqFilterPer; ++j) {
      key[j] = score_key(sc[j]);
      kmin = val[j] ? min(kmin, key[j]) : kmin;
      kmax = val[j] ? max(kmax, key[j]) : kmax;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, kWave));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, kWave));
    }
    if (lane == 0) {
      sh.kmin[tid / kWave] = kmin;
      sh.kmax[tid / kWave] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kPqFilterWaves; ++w) {
      kmin = min(kmin, sh.kmin[w]);
      kmax = max(kmax, sh.kmax[w]);
    }
    const uint32_t diff = kmin ^ kmax;
    int top = diff ? 31 - __clz(diff) : -1;           // highest undecided bit
    uint32_t pmask = top >= 0 ? ~((2u << top) - 1u) : 0xFFFFFFFFu;
    if (top == 31) pmask = 0u;
    uint32_t prefix = kmin & pmask;
    for (int d = 0; top >= 0; ++d) {
      const int width = top >= 7 ? 8 : top + 1;
      const int shift = top - width + 1, hb = d & 1;
      const uint32_t dm = (1u << width) - 1u;
#pragma unroll
      for (int j = 0; j < kPqFilterPer; ++j)
        if (val[j] && (key[j] & pmask) == prefix) atomicAdd(&sh.hist[hb][(key[j] >> shift) & dm], 1u);
      if (tid < 256) sh.hist[hb ^ 1][tid] = 0u;
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins 4l .. 4l + 3; the digit holding the need-th largest
        int cnt = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) cnt += (int)sh.hist[hb][4 * lane + b];
        const int below = wave_incl_scan(cnt, lane) - cnt;
        const int tot = __shfl(below + cnt, kWave - 1, kWave);
        int above = tot - below - cnt;
        if (above < need && above + cnt >= need) {
          for (int b = 3; b >= 0; --b) {
            const int h = (int)sh.hist[hb][4 * lane + b];
            if (above + h >= need) {
              sh.digit[hb] = 4 * lane + b;
              sh.above[hb] = above;
              break;
            }
            above += h;
          }
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh.digit[hb] << shift;
      pmask |= dm << shift;
      need -= sh.above[hb];
      top -= width;
    }
    theta = (double)pq_key_score(prefix) - sd;
  }
  // keep hits, and misses at or above theta; compact in candidate order (the
  // kept count in the low 16 bits of the scanned value, kept misses above)
  bool keep[kPqFilterPer];
  int nk = 0, nm = 0;
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j) {
    keep[j] = val[j] && (res[j] || (double)sc[j] >= theta);
    nk += keep[j];
    nm += keep[j] && !res[j];
  }
  int tot;
  const int ex = pq_block_scan(nk | (nm << 16), sh.ired, &tot);
  const int total = tot & 0xFFFF, misses = tot >> 16;
  int pos = ex & 0xFFFF;
  int32_t* out = a.kept + (size_t)r * a.cap;
#pragma unroll
  for (int j = 0; j < kPqFilterPer; ++j)
    if (keep[j]) out[pos++] = tok[j];
  for (int i = total + tid; i < a.cap; i += kPqFilterThreads) out[i] = -1;
  if (tid == 0) {
    a.kept_counts[r] = total;
    if (a.misses_kept) a.misses_kept[r] = misses;
  }
}

hipError_t launch_pq_filter(const PqFilterArgs& a, int batch, hipStream_t st) {
  hipLaunchKernelGGL(pq_filter_kernel, dim3(batch), dim3(kPqFilterThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ls

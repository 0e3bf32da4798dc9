// Split-K gather attention over the selected blocks of a paged KV cache, and
// the log-sum-exp combine of the splits.
//
// Vortex post, block top-k equation: o = softmax(q K_I^T / sqrt(d)) V_I over
// the tokens of the selected blocks I. The combine is the log-sum-exp merge
// of attention results over disjoint token sets (ByteCross paper, "Where
// Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding", App. A,
// which merges its sink call with its window call this way).
//
// Grid: (split, kv head, request). A split is a contiguous, balanced slice of
// the request's selection list for that kv head, at most kAttnBlocksPerSplit
// blocks, so one workgroup issues every K and V load of its slice before it
// computes (up to 64 KB in flight per workgroup at D = 128). A (page, head)
// tile is page_size x D contiguous bf16; thread t loads 16 bytes (8 dims of
// one token row) of each K and V tile, so a wave instruction reads 1 KB
// contiguous and the workgroup reads a whole 4 KB tile per instruction.
// There is no reuse of K/V across threads, so the data goes straight to
// registers; LDS is used only to merge the per-row softmax states at the end.
//
// Each group of D/8 lanes owns one token row: the G query heads' logits are
// v_dot2 partial sums reduced over those lanes, and each lane then keeps a
// private online-softmax state (running max m, sum l, and o over its 8 dims)
// per head, in the log2 domain (logits pre-scaled by sm_scale * log2 e, so
// every exponential is one exp2). States of all rows are merged in LDS and
// the split's (m, l, unnormalised o) is written to the partial buffer.
#include "ls_internal.h"

namespace ls {

constexpr float kLn2 = 0.6931471805599453f;

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

template <int D, int G>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  constexpr int P = 16;                 // tokens per block (page)
  constexpr int LPR = D / 8;            // lanes per token row
  constexpr int RPW = kWave / LPR;      // rows per wave
  constexpr int ROWS = 4 * RPW;         // rows per workgroup round
  constexpr int BPR = ROWS / P;         // blocks per round (1 at D=128, 2 at D=64)
  constexpr int CH = kAttnBlocksPerSplit / BPR;  // rounds per split
  constexpr float kNegInf = -__builtin_huge_valf();

  __shared__ float sm_acc[ROWS][G][D];
  __shared__ float sm_m[ROWS][G];
  __shared__ float sm_l[ROWS][G];

  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = wave * RPW + lane / LPR;
  const int c = lane % LPR;
  const int bir = row / P, slot = row % P;
  const int HKV = a.num_kv_heads;

  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  int cnt = geo.nb;
  const int32_t* selrow = nullptr;
  if (a.selected) {
    cnt = a.selected_count[(size_t)r * HKV + g];
    cnt = cnt < 0 ? 0 : (cnt > a.max_selected ? a.max_selected : cnt);
    selrow = a.selected + ((size_t)r * HKV + g) * a.max_selected;
  }
  const int S = a.num_splits;
  const int lo = (int)(((long long)s * cnt) / S);
  const int hi = (int)(((long long)(s + 1) * cnt) / S);

  // the group's query heads, 8 dims of each, as bf16 pairs
  uint32_t qv[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = ldg16(a.q + ((size_t)r * a.num_q_heads + g * G + h) * D + c * 8);
    qv[h][0] = t.x; qv[h][1] = t.y; qv[h][2] = t.z; qv[h][3] = t.w;
  }

  // issue every K and V load of this split
  uint4 kr[CH], vr[CH];
  bool ok[CH];
  const int32_t* pages = a.b.indices + geo.page_base;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int idx = lo + i * BPR + bir;
    bool v = idx < hi;
    int blk = v ? (selrow ? selrow[idx] : idx) : 0;
    v = v && blk >= 0 && blk < geo.nb && blk * P + slot < geo.L;
    int page = v ? pages[blk] : 0;
    v = v && page >= 0 && page < a.b.num_pages;
    ok[i] = v;
    const size_t off = (((size_t)page * HKV + g) * P + slot) * D + c * 8;
    kr[i] = v ? ldg16(a.k_pool + off) : make_uint4(0, 0, 0, 0);
    vr[i] = v ? ldg16(a.v_pool + off) : make_uint4(0, 0, 0, 0);
  }

  // logits (log2 domain), reduced over the row's lanes
  float z[CH][G];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
#pragma unroll
    for (int h = 0; h < G; ++h) z[i][h] = dot8(qv[h], kr[i], 0.0f);
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] += __shfl_xor(z[i][h], o, kWave);
    }
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      z[i][h] = ok[i] ? z[i][h] * a.sm_scale_log2 : kNegInf;
      mx = fmaxf(mx, z[i][h]);
    }
    m[h] = mx;
    l[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.0f;
    if (mx != kNegInf) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float p = ok[i] ? exp2f(z[i][h] - mx) : 0.0f;
        l[h] += p;
        const uint4 v = vr[i];
        acc[h][0] += p * bf16_lo(v.x); acc[h][1] += p * bf16_hi(v.x);
        acc[h][2] += p * bf16_lo(v.y); acc[h][3] += p * bf16_hi(v.y);
        acc[h][4] += p * bf16_lo(v.z); acc[h][5] += p * bf16_hi(v.z);
        acc[h][6] += p * bf16_lo(v.w); acc[h][7] += p * bf16_hi(v.w);
      }
    }
  }

  // merge the ROWS row states
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int d = 0; d < 8; ++d) sm_acc[row][h][c * 8 + d] = acc[h][d];
    if (c == 0) { sm_m[row][h] = m[h]; sm_l[row][h] = l[h]; }
  }
  __syncthreads();
  float* part = a.partials + (((size_t)r * a.num_q_heads + g * G) * S + s) * (D + 2);
  for (int o = tid; o < G * D; o += 256) {
    const int h = o / D, d = o % D;
    float M = kNegInf;
#pragma unroll 4
    for (int w = 0; w < ROWS; ++w) M = fmaxf(M, sm_m[w][h]);
    float O = 0.0f, Ls = 0.0f;
    if (M != kNegInf) {
      for (int w = 0; w < ROWS; ++w) {
        const float e = exp2f(sm_m[w][h] - M);  // rows with m = -inf give 0
        O += e * sm_acc[w][h][d];
        Ls += e * sm_l[w][h];
      }
    }
    float* ph = part + (size_t)h * S * (D + 2);
    ph[d] = O;
    if (d == 0) { ph[D] = M; ph[D + 1] = Ls; }
  }
}

// One wave per (request, query head): merge the S split partials in split
// order, normalise, round once to the output dtype.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr float kNegInf = -__builtin_huge_valf();
  constexpr int DPL = D / kWave;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nitems = a.b.batch * a.num_q_heads;
  if (item >= nitems) return;
  const int S = a.num_splits;
  const float* part = a.partials + (size_t)item * S * (D + 2);
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[(size_t)s * (D + 2) + D]);
  float O[DPL], Ls = 0.0f;
#pragma unroll
  for (int j = 0; j < DPL; ++j) O[j] = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float* ps = part + (size_t)s * (D + 2);
      const float e = exp2f(ps[D] - M);
      Ls += e * ps[D + 1];
#pragma unroll
      for (int j = 0; j < DPL; ++j) O[j] += e * ps[lane + j * kWave];
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

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.num_splits, a.num_kv_heads, a.b.batch);
  hipLaunchKernelGGL((attn_split_kernel<D, 4>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items = a.b.batch * a.num_q_heads;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((items + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.head_dim == 128) return launch_d<128>(a, st);
  return launch_d<64>(a, st);
}

}  // namespace ls

// Sparse multi-head latent attention over selected tokens (decode step).
//
// Every query head h of request r attends the single shared latent head over
// the selected tokens T (Vortex, "Designing for a new architecture": keys are
// the whole latent row -- compressed content and rope part -- and values its
// first v_dim entries):
//     z_t = sm_scale * q[r][h] . c_t[0:576],  o_h = sum_t softmax(z)_t c_t[0:512].
// The selection is split over workgroups (tokens [s*kMlaSplitTokens, +)) and
// the partial softmax states are merged by log-sum-exp in a second kernel,
// in split order (deterministic).
//
// Workgroup (r, 16-head group, split), 4 waves. Per 32-token tile, staged in
// LDS from contiguous 1152-byte token rows:
//  * logits z^T = C . q^T on the matrix cores (16x16x32 bf16): A = latent rows
//    (16 tokens x 32 dims), B = q^T (32 dims x 16 heads); the 18 k-steps are
//    split over the 4 waves and the partial logits are summed through LDS, so
//    every wave ends up with lane i holding head i%16, tokens 4(i/16)+j of
//    both 16-token halves;
//  * online softmax per head (every wave keeps the same state);
//  * o += P . V with wave w owning output dims [128w, 128w+128): A = P (16
//    heads x 32 tokens, split into bf16 parts hi + lo (+ lo2 for fp32 output)
//    for fp32-level accuracy), B = V columns read from the LDS tile in the
//    token order of P's k-slices.
#include "dev_mfma.h"
#include "ls_internal.h"

namespace ls {

constexpr int kMlaDk = 576, kMlaDv = 512;
constexpr int kMlaPartStride = kMlaDv + 4;   // o[512], m, l, pad: 16-byte aligned rows
constexpr int kMlaThreads = 256, kMlaWaves = 4;
constexpr int kMlaHeadsPerWg = 16;
constexpr int kMlaTile = 32;                           // tokens per LDS tile
constexpr int kMlaRowWords = kMlaDk / 2 + 4;           // 1168-byte padded rows (16-byte aligned)
constexpr int kMlaChunks = kMlaTile * (kMlaDk / 8);    // 16-byte chunks per tile
constexpr int kMlaChunksPerThread = kMlaChunks / kMlaThreads;
static_assert(kMlaChunks % kMlaThreads == 0, "tile chunks per thread");

struct MlaLds {
  alignas(16) uint32_t tile[kMlaTile * kMlaRowWords];
  f32x4_t red[kMlaWaves][2][kWave];
  int rowoff[kMlaSplitTokens];   // token row index in the pool (page * P + slot), -1 = skip
};

__device__ __forceinline__ uint32_t mla_bf16_split(float x, float* rest) {
  const uint32_t b = f32_to_bf16_rne(x);
  *rest = x - __uint_as_float(b << 16);
  return b;
}

// two workgroups per CU (<= 256 registers per lane)
__global__ __launch_bounds__(kMlaThreads, 2) void mla_split_kernel(MlaArgs a) {
  __shared__ MlaLds sh;
  const int S = a.num_splits;
  const int nrs = a.b.batch * S;
  const int rs = blockIdx.x % nrs, hg = blockIdx.x / nrs;   // same (r, s): same XCD
  const int r = rs / S, s = rs % S;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int P = a.b.page_size;
  const int H = a.num_q_heads;

  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  int cnt = a.selected_count ? a.selected_count[r] : geo.L;
  cnt = cnt < 0 ? 0 : (cnt > a.max_selected && a.selected ? a.max_selected : cnt);
  const int p0 = s * kMlaSplitTokens;
  int ntok = cnt - p0;
  ntok = ntok < 0 ? 0 : (ntok > kMlaSplitTokens ? kMlaSplitTokens : ntok);
  for (int i = tid; i < kMlaSplitTokens; i += kMlaThreads) {
    int off = -1;
    if (i < ntok) {
      const int t = a.selected ? a.selected[(size_t)r * a.max_selected + p0 + i] : p0 + i;
      if (t >= 0 && t < geo.L) {
        const int pg = a.b.indices[geo.page_base + t / P];
        if (pg >= 0 && pg < a.b.num_pages) off = pg * P + t % P;
      }
    }
    sh.rowoff[i] = off;
  }
  // q^T operand for this wave's k-steps: head 16hg + col, dims 32k + 8kq
  const int ks0 = wave < 2 ? 5 * wave : 10 + 4 * (wave - 2);
  const int nks = wave < 2 ? 5 : 4;
  uint4 qb[5];
  const uint16_t* qh = a.q + ((size_t)r * H + kMlaHeadsPerWg * hg + col) * kMlaDk + 8 * kq;
#pragma unroll
  for (int k = 0; k < 5; ++k) qb[k] = k < nks ? ldg16(qh + 32 * (ks0 + k)) : make_uint4(0, 0, 0, 0);
  __syncthreads();

  const bool out32 = a.out_dtype == LS_DTYPE_FP32;
  const int ntiles = (ntok + kMlaTile - 1) / kMlaTile;
  // tile loads: chunk c = tid + 256 i -> token c / 72, 16 bytes at 8 (c % 72);
  // two tiles of loads are in flight (register buffers A and B)
  auto issue = [&](int t, uint4* ld) {
#pragma unroll
    for (int i = 0; i < kMlaChunksPerThread; ++i) {
      const int c = tid + kMlaThreads * i;
      const int tok = t * kMlaTile + c / (kMlaDk / 8);
      const int off = (t < ntiles && tok < ntok) ? sh.rowoff[tok] : -1;
      ld[i] = ldg16_stream(a.latent + (size_t)(uint32_t)(off >= 0 ? off : 0) * kMlaDk + 8 * (c % (kMlaDk / 8)));
    }
  };
  f32x4_t o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kNegInf, l = 0.0f;   // state of head `col`
  auto tile_step = [&](int t, uint4* ld) {
    // stage tile t, then start loading tile t + 2 into the same registers
#pragma unroll
    for (int i = 0; i < kMlaChunksPerThread; ++i) {
      const int c = tid + kMlaThreads * i;
      *reinterpret_cast<uint4*>(sh.tile + (c / (kMlaDk / 8)) * kMlaRowWords + 4 * (c % (kMlaDk / 8))) = ld[i];
    }
    __syncthreads();
    issue(t + 2, ld);
    // partial logits over this wave's k-steps: rows = tokens, cols = heads
    f32x4_t z0 = {0.0f, 0.0f, 0.0f, 0.0f}, z1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      if (k < nks) {
        const int w0 = 16 * (ks0 + k) + 4 * kq;
        const uint4 a0 = *reinterpret_cast<const uint4*>(sh.tile + col * kMlaRowWords + w0);
        const uint4 a1 = *reinterpret_cast<const uint4*>(sh.tile + (16 + col) * kMlaRowWords + w0);
        z0 = mfma_16x16x32(a0, qb[k], z0);
        z1 = mfma_16x16x32(a1, qb[k], z1);
      }
    }
    sh.red[wave][0][lane] = z0;
    sh.red[wave][1][lane] = z1;
    __syncthreads();
    f32x4_t zs0 = sh.red[0][0][lane], zs1 = sh.red[0][1][lane];
#pragma unroll
    for (int w = 1; w < kMlaWaves; ++w) {
      const f32x4_t x0 = sh.red[w][0][lane], x1 = sh.red[w][1][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) { zs0[i] += x0[i]; zs1[i] += x1[i]; }
    }
    // lane: head col; tokens 4kq + i (half 0) and 16 + 4kq + i (half 1)
    float z[8], bm = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t0 = t * kMlaTile + 4 * kq + i, t1 = t0 + 16;
      z[i] = (t0 < ntok && sh.rowoff[t0] >= 0) ? zs0[i] * a.sm_scale_log2 : kNegInf;
      z[4 + i] = (t1 < ntok && sh.rowoff[t1] >= 0) ? zs1[i] * a.sm_scale_log2 : kNegInf;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) bm = fmaxf(bm, z[i]);
    float lo, hi;
    xor_pair<16>(bm, lo, hi);
    bm = fmaxf(lo, hi);
    xor_pair<32>(bm, lo, hi);
    bm = fmaxf(lo, hi);
    const float mn = fmaxf(m, bm);
    const float alpha = mn == kNegInf ? 1.0f : exp2f(m - mn);
    float p[8], ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = z[i] == kNegInf ? 0.0f : exp2f(z[i] - mn);
      ps += p[i];
    }
    ps = xor_pair_sum<16>(ps);
    ps = xor_pair_sum<32>(ps);
    l = l * alpha + ps;
    m = mn;
    // o rows are heads 4kq + i: their alphas live in lanes 4kq + i
    if (__ballot(alpha != 1.0f)) {
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * kq + i);
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= ar[i];
    }
    // P (A operand: row = head col, k-slice kq = tokens 4kq+i, 16+4kq+i)
    uint32_t h16[8], l16[8], m16[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r1, r2;
      h16[i] = mla_bf16_split(p[i], &r1);
      l16[i] = mla_bf16_split(r1, &r2);
      m16[i] = f32_to_bf16_rne(r2);
    }
    const uint4 ph = make_uint4(h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16),
                                h16[4] | (h16[5] << 16), h16[6] | (h16[7] << 16));
    const uint4 pl = make_uint4(l16[0] | (l16[1] << 16), l16[2] | (l16[3] << 16),
                                l16[4] | (l16[5] << 16), l16[6] | (l16[7] << 16));
    const uint4 pm = make_uint4(m16[0] | (m16[1] << 16), m16[2] | (m16[3] << 16),
                                m16[4] | (m16[5] << 16), m16[6] | (m16[7] << 16));
    // o += P . V over this wave's 128 dims; B = V[the same 8 tokens][dim]
    const uint16_t* tb = reinterpret_cast<const uint16_t*>(sh.tile);
    constexpr int RS = 2 * kMlaRowWords;   // row stride in bf16 elements
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint16_t* c = tb + 4 * kq * RS + 128 * wave + 16 * n + col;
      const uint4 vb = make_uint4((uint32_t)c[0] | ((uint32_t)c[RS] << 16),
                                  (uint32_t)c[2 * RS] | ((uint32_t)c[3 * RS] << 16),
                                  (uint32_t)c[16 * RS] | ((uint32_t)c[17 * RS] << 16),
                                  (uint32_t)c[18 * RS] | ((uint32_t)c[19 * RS] << 16));
      o[n] = mfma_16x16x32(ph, vb, o[n]);
      o[n] = mfma_16x16x32(pl, vb, o[n]);
      if (out32) o[n] = mfma_16x16x32(pm, vb, o[n]);
    }
    __syncthreads();   // the tile and the logit partials are rewritten next
  };
  uint4 ldA[kMlaChunksPerThread], ldB[kMlaChunksPerThread];
  issue(0, ldA);
  issue(1, ldB);
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(t, ldA);
    if (t + 1 < ntiles) tile_step(t + 1, ldB);
  }
  // partial state: o rows = heads 4kq + i, column = dim 128 wave + 16 n + col
  float* part = a.partials + (((size_t)r * H + kMlaHeadsPerWg * hg) * S + s) * (kMlaPartStride);
  const size_t hstride = (size_t)S * (kMlaPartStride);
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(4 * kq + i) * hstride + 128 * wave + 16 * n + col] = o[n][i];
  if (wave == 0 && kq == 0) {
    part[col * hstride + kMlaDv] = m;
    part[col * hstride + kMlaDv + 1] = l;
  }
}

// One (request, head) row per 128-thread group: merge the S split states in
// split order.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a) {
  const int row = blockIdx.x * 2 + (threadIdx.x >> 7);
  const int t = threadIdx.x & 127;
  if (row >= a.b.batch * a.num_q_heads) return;
  const int S = a.num_splits;
  const float* part = a.partials + (size_t)row * S * (kMlaPartStride);
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[s * (kMlaPartStride) + kMlaDv]);
  float O[4] = {0.0f, 0.0f, 0.0f, 0.0f}, Ls = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float* ps = part + s * (kMlaPartStride);
      const float f = exp2f(ps[kMlaDv] - M);   // splits with m = -inf give 0
      Ls += f * ps[kMlaDv + 1];
      const float4 v = *reinterpret_cast<const float4*>(ps + 4 * t);
      O[0] += f * v.x; O[1] += f * v.y; O[2] += f * v.z; O[3] += f * v.w;
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  const size_t base = (size_t)row * kMlaDv + 4 * t;
  if (a.out_dtype == LS_DTYPE_FP32) {
    float* out = reinterpret_cast<float*>(a.out) + base;
    *reinterpret_cast<float4*>(out) = make_float4(O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv);
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + base;
    const uint2 pk = make_uint2((uint32_t)f32_to_bf16_rne(O[0] * inv) | ((uint32_t)f32_to_bf16_rne(O[1] * inv) << 16),
                                (uint32_t)f32_to_bf16_rne(O[2] * inv) | ((uint32_t)f32_to_bf16_rne(O[3] * inv) << 16));
    *reinterpret_cast<uint2*>(out) = pk;
  }
  if (a.lse && t == 0)
    a.lse[row] = (M == kNegInf || !(Ls > 0.0f)) ? kNegInf : (M + log2f(Ls)) * kLn2;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t st) {
  const int nwg = a.b.batch * a.num_splits * (a.num_q_heads / kMlaHeadsPerWg);
  hipLaunchKernelGGL(mla_split_kernel, dim3(nwg), dim3(kMlaThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.b.batch * a.num_q_heads;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((rows + 1) / 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ls

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
// Workgroup (r, 32 heads, split), 8 waves; the latent rows of a 64-token
// tile are staged once in LDS (contiguous 1152-byte token rows) and shared by
// both 16-head tiles:
//  * logits z^T = C . q^T on the matrix cores (16x16x32 bf16): A = latent rows
//    (16 tokens x 32 dims), B = q^T (32 dims x 16 heads); the 18 k-steps are
//    split over the 4 waves of a head tile and their partial logits summed
//    through LDS, so each wave ends up with lane i holding head i%16, tokens
//    4(i/16)+j of each 16-token row tile;
//  * online softmax per head (the 4 waves of a head tile keep the same state);
//  * o += P . V with the 4 waves of a head tile owning 128 output dims each:
//    A = P (16 heads x 32 tokens, split into bf16 parts hi + lo (+ lo2 for
//    fp32 output) for fp32-level accuracy), B = V columns read from the LDS
//    tile in the token order of P's k-slices.
#include "dev_mfma.h"
#include "ls_internal.h"

namespace ls {

constexpr int kMlaDk = 576, kMlaDv = 512;
// Workgroup shape (measured on MI355X): head tiles of 16 heads per workgroup
// (4 waves each) and 16-token row tiles per LDS tile.
#ifndef LS_MLA_HEAD_TILES
#define LS_MLA_HEAD_TILES 2
#endif
#ifndef LS_MLA_ROW_TILES
#define LS_MLA_ROW_TILES 4
#endif
constexpr int kMlaHT = LS_MLA_HEAD_TILES;              // 16-head tiles per workgroup
constexpr int kMlaRT = LS_MLA_ROW_TILES;               // 16-token row tiles per LDS tile
constexpr int kMlaWaves = 4 * kMlaHT, kMlaThreads = kMlaWaves * kWave;
constexpr int kMlaHeadsPerWg = 16 * kMlaHT;
constexpr int kMlaTile = 16 * kMlaRT;                  // tokens per LDS tile
constexpr int kMlaRowWords = kMlaDk / 2 + 4;           // 1168-byte padded rows (16-byte aligned)
constexpr int kMlaChunks = kMlaTile * (kMlaDk / 8);    // 16-byte chunks per tile
constexpr int kMlaChunksPerThread = kMlaChunks / kMlaThreads;
static_assert(kMlaChunksPerThread <= 32, "one mask bit per chunk");
static_assert(kMlaChunks % kMlaThreads == 0, "tile chunks per thread");
static_assert(kMlaSplitTokens % 64 == 0 && kMlaSplitTokens % kMlaTile == 0, "whole tiles per split");
static_assert(kMlaRT % 2 == 0, "P . V k-steps of 32 tokens");

// Byte offset of the o partials in the workspace: after the (m, l) pairs of
// every (request, head, split) row, 256-byte aligned.
__device__ __forceinline__ size_t mla_o_offset(const MlaArgs& a) {
  const size_t ml = (size_t)a.b.batch * a.num_q_heads * a.num_splits * 2 * sizeof(float);
  return (ml + 255) / 256 * 256;
}

struct MlaLds {
  alignas(16) uint32_t tile[kMlaTile * kMlaRowWords];
  f32x4_t red[kMlaWaves][kMlaRT][kWave];   // partial logits: wave, 16-token row tile, lane
  int rowoff[kMlaSplitTokens];             // token row index in the pool (page * P + slot), -1 = skip
  unsigned long long valid[kMlaSplitTokens / 64];   // bit = token row present
};

// Workgroup (request r, 16 kMlaHT heads, split s), 4 kMlaHT waves. Wave w
// works on head tile w / 4 (16 heads): the QK^T k-steps of quarter w % 4 (5,
// 5, 4, 4 of the 18), summed with the other three waves of its head tile
// through LDS, and the output dims [128 (w % 4), + 128) of P . V.
#ifdef LS_MLA_WAVES_PER_EU
#define LS_MLA_WPE __attribute__((amdgpu_waves_per_eu(LS_MLA_WAVES_PER_EU)))
#else
#define LS_MLA_WPE
#endif
__global__ __launch_bounds__(kMlaThreads) LS_MLA_WPE void mla_split_kernel(MlaArgs a) {
  __shared__ MlaLds sh;
  const int S = a.num_splits;
  const int nrs = a.b.batch * S;
  const int rs = blockIdx.x % nrs, hg = blockIdx.x / nrs;   // same (r, s): same XCD
  const int r = rs / S, s = rs % S;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int ht = wave >> 2, sub = wave & 3;
  const int P = a.b.page_size;
  const int H = a.num_q_heads;

  // q^T operand of this wave's k-steps: head 16 (kMlaHT hg + ht) + col, dims
  // 32k + 8kq (issued first: independent of the selection)
  const int ks0 = sub < 2 ? 5 * sub : 10 + 4 * (sub - 2);
  const int nks = sub < 2 ? 5 : 4;
  const int head0 = kMlaHeadsPerWg * hg + 16 * ht;
  uint4 qb[5];
  const uint16_t* qh = a.q + ((size_t)r * H + head0 + col) * kMlaDk + 8 * kq;
#pragma unroll
  for (int k = 0; k < 5; ++k) qb[k] = k < nks ? ldg16(qh + 32 * (ks0 + k)) : make_uint4(0, 0, 0, 0);

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
    const unsigned long long vb = __ballot(off >= 0);   // a wave = 64 consecutive tokens
    if ((i & (kWave - 1)) == 0) sh.valid[i / kWave] = vb;
  }
  __syncthreads();

  const bool out32 = a.out_dtype == LS_DTYPE_FP32;
  const int ntiles = (ntok + kMlaTile - 1) / kMlaTile;
  // tile loads: chunk c = tid + kMlaThreads i -> token c / 72, 16 bytes at
  // 8 (c % 72); one tile of loads is in flight while the staged one is used.
  // vm: bit i set when chunk i belongs to a selected token (the others read
  // row 0 and are zeroed when staged: their weights are 0, but 0 * NaN would
  // reach the output)
  auto issue = [&](int t, uint4* ld, uint32_t& vm) {
    vm = 0u;
#pragma unroll
    for (int i = 0; i < kMlaChunksPerThread; ++i) {
      const int c = tid + kMlaThreads * i;
      const int tok = t * kMlaTile + c / (kMlaDk / 8);
      const int off = (t < ntiles && tok < ntok) ? sh.rowoff[tok] : -1;
      vm |= off >= 0 ? (1u << i) : 0u;
      ld[i] = ldg16_stream(a.latent + (size_t)(uint32_t)(off >= 0 ? off : 0) * kMlaDk + 8 * (c % (kMlaDk / 8)));
    }
  };
  f32x4_t o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kNegInf, l = 0.0f;   // state of head head0 + col
  constexpr int RS = 2 * kMlaRowWords;   // LDS row stride in bf16 elements
  constexpr uint32_t kAllChunks = (1u << kMlaChunksPerThread) - 1u;
  auto tile_step = [&](int t, uint4* ld, uint32_t& vm) {
    // stage tile t, then start loading tile t + 1 into the same registers
    if (vm != kAllChunks) {
#pragma unroll
      for (int i = 0; i < kMlaChunksPerThread; ++i)
        if (!((vm >> i) & 1u)) ld[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kMlaChunksPerThread; ++i) {
      const int c = tid + kMlaThreads * i;
      *reinterpret_cast<uint4*>(sh.tile + (c / (kMlaDk / 8)) * kMlaRowWords + 4 * (c % (kMlaDk / 8))) = ld[i];
    }
    __syncthreads();
    issue(t + 1, ld, vm);
    // partial logits over this wave's k-steps, kMlaRT row tiles of 16 tokens
    f32x4_t z[kMlaRT];
#pragma unroll
    for (int j = 0; j < kMlaRT; ++j) z[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      if (k < nks) {
        const int w0 = 16 * (ks0 + k) + 4 * kq;
#pragma unroll
        for (int j = 0; j < kMlaRT; ++j) {
          const uint4 av = *reinterpret_cast<const uint4*>(sh.tile + (16 * j + col) * kMlaRowWords + w0);
          z[j] = mfma_16x16x32(av, qb[k], z[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMlaRT; ++j) sh.red[wave][j][lane] = z[j];
    __syncthreads();
    // full logits of head tile ht: lane = head col, tokens 16 j + 4 kq + i
    const int tp = t * kMlaTile;   // first token of the tile in the split
    const unsigned long long vbits = (sh.valid[tp >> 6] >> (tp & 63)) >> (4 * kq);
    float zz[4 * kMlaRT], bm = kNegInf;
#pragma unroll
    for (int j = 0; j < kMlaRT; ++j) {
      f32x4_t acc = sh.red[4 * ht][j][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4_t x = sh.red[4 * ht + w][j][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += x[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zz[4 * j + i] = ((vbits >> (16 * j + i)) & 1ull) ? acc[i] * a.sm_scale_log2 : kNegInf;
        bm = fmaxf(bm, zz[4 * j + i]);
      }
    }
    float lo, hi;
    xor_pair<16>(bm, lo, hi);
    bm = fmaxf(lo, hi);
    xor_pair<32>(bm, lo, hi);
    bm = fmaxf(lo, hi);
    const float mn = fmaxf(m, bm);
    // exp2 of values <= 0 with -inf -> 0 (mn = -inf: nothing seen yet, all 0)
    const float mref = mn == kNegInf ? 0.0f : mn;
    const float alpha = mn == kNegInf ? 1.0f : exp2_fast(m - mref);
    float p[4 * kMlaRT], ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * kMlaRT; ++i) {
      p[i] = exp2_fast(zz[i] - mref);
      ps += p[i];
    }
    ps = xor_pair_sum<16>(ps);
    ps = xor_pair_sum<32>(ps);
    l = l * alpha + ps;
    m = mn;
    // o rows are heads 4kq + i of the tile: their alphas live in lanes 4kq + i
    if (__ballot(alpha != 1.0f)) {
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * kq + i);
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= ar[i];
    }
    // P . V in k-steps of 32 tokens: step js covers row tiles 2js and
    // 2js + 1; lane's k-slice = tokens 4kq + i of each (P as A: row = head col)
#pragma unroll
    for (int js = 0; js < kMlaRT / 2; ++js) {
      // p = hi + lo (+ lo2) in bf16 parts, two tokens per conversion
      uint32_t hw[4], lw[4], mw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = p[8 * js + 2 * i], y = p[8 * js + 2 * i + 1];
        bf16x2_split(x, y, &hw[i]);
        bf16x2_split(x, y, &lw[i]);
        mw[i] = out32 ? pack_bf16x2(x, y) : 0u;
      }
      const uint4 ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      const uint4 pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      const uint4 pm = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      // V as B operand via transpose reads: this lane addresses row
      // 32 js + 4 kq + (col / 4) (and + 16) at columns 4 (col % 4) of the
      // 16-dim tile, and receives column col of rows 32 js + 4 kq + 0..3 (+ 16)
      const uint16_t* tb = reinterpret_cast<const uint16_t*>(sh.tile) +
                           (32 * js + 4 * kq + (col >> 2)) * RS + 128 * sub + 4 * (col & 3);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint2 v0 = lds_read_tr16(tb + 16 * n);
        const uint2 v1 = lds_read_tr16(tb + 16 * RS + 16 * n);
        const uint4 vb = make_uint4(v0.x, v0.y, v1.x, v1.y);
        o[n] = mfma_16x16x32(ph, vb, o[n]);
        o[n] = mfma_16x16x32(pl, vb, o[n]);
        if (out32) o[n] = mfma_16x16x32(pm, vb, o[n]);
      }
    }
    __syncthreads();   // the tile and the logit partials are rewritten next
  };
  uint4 ldA[kMlaChunksPerThread];
  uint32_t vmA;
  issue(0, ldA, vmA);
  for (int t = 0; t < ntiles; ++t) tile_step(t, ldA, vmA);
  // partial state: (m, l) per head, and o, rows = heads 4kq + i of the tile,
  // column = dim 128 sub + 16 n + col: unnormalised fp32 for fp32 output,
  // normalised (o / l, bounded by the largest |v|) bf16 for bf16 output
  const size_t prow = ((size_t)r * H + head0) * S + s;   // (head0, s) partial row
  float* ml = a.partials;
  if (sub == 0 && kq == 0) {
    ml[(prow + (size_t)col * S) * 2] = m;
    ml[(prow + (size_t)col * S) * 2 + 1] = l;
  }
  char* obase = reinterpret_cast<char*>(a.partials) + mla_o_offset(a);
  if (out32) {
    float* po = reinterpret_cast<float*>(obase) + prow * kMlaDv;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        po[(size_t)(4 * kq + i) * S * kMlaDv + 128 * sub + 16 * n + col] = o[n][i];
  } else {
    uint16_t* po = reinterpret_cast<uint16_t*>(obase) + prow * kMlaDv;
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l, 4 * kq + i);
      inv[i] = li > 0.0f ? 1.0f / li : 0.0f;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        po[(size_t)(4 * kq + i) * S * kMlaDv + 128 * sub + 16 * n + col] = f32_to_bf16_rne(o[n][i] * inv[i]);
  }
}

// One (request, head) row per 128-thread group: merge the S split states in
// split order.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a) {
  const int row = blockIdx.x * 2 + (threadIdx.x >> 7);
  const int t = threadIdx.x & 127;
  if (row >= a.b.batch * a.num_q_heads) return;
  const int S = a.num_splits;
  const bool out32 = a.out_dtype == LS_DTYPE_FP32;
  const float* ml = a.partials + (size_t)row * S * 2;
  const char* obase = reinterpret_cast<const char*>(a.partials) + mla_o_offset(a);
  // 8 splits per round; the o rows do not depend on the running maximum, so
  // the first round's are issued before the (m, l) pairs and all of them
  // arrive in one memory round trip (splits past S re-read split S - 1 and
  // get weight 0)
  constexpr int U = 8;
  float4 vf[U];
  uint2 vb[U];
  auto load_o = [&](int s0) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int s = s0 + j < S ? s0 + j : S - 1;
      const size_t oi = ((size_t)row * S + s) * kMlaDv + 4 * t;
      if (out32) vf[j] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(obase) + oi);
      else vb[j] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(obase) + oi);
    }
  };
  load_o(0);
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float O[4] = {0.0f, 0.0f, 0.0f, 0.0f}, Ls = 0.0f;
  if (M != kNegInf) {
    for (int s0 = 0; s0 < S; s0 += U) {
      if (s0 > 0) load_o(s0);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int s = s0 + j < S ? s0 + j : S - 1;
        const float f = s0 + j < S ? exp2_fast(ml[2 * s] - M) : 0.0f;   // splits with m = -inf give 0
        const float ls = ml[2 * s + 1];
        Ls += f * ls;
        if (out32) {
          O[0] += f * vf[j].x; O[1] += f * vf[j].y; O[2] += f * vf[j].z; O[3] += f * vf[j].w;
        } else {
          const float w = f * ls;   // the split's o was stored divided by its l
          O[0] += w * bf16_lo(vb[j].x); O[1] += w * bf16_hi(vb[j].x);
          O[2] += w * bf16_lo(vb[j].y); O[3] += w * bf16_hi(vb[j].y);
        }
      }
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  const size_t base = (size_t)row * kMlaDv + 4 * t;
  if (out32) {
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
  const int nwg = a.b.batch * a.num_splits * (a.num_q_heads / kMlaHeadsPerWg);   // H % 32 == 0
  hipLaunchKernelGGL(mla_split_kernel, dim3(nwg), dim3(kMlaThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.b.batch * a.num_q_heads;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((rows + 1) / 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ls

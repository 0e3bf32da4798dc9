// Learned-indexer kernels: MFMA scoring of tokens (fp8 keys) or blocks
// (bf16 block-mean keys), and the multi-workgroup token top-k (see
// dev_indexer.h for the method).
#include "dev_indexer.h"
#include "dev_mfma.h"

namespace ls {

// ------------------------------------------------------------- scoring ----

// Per-mode tile geometry: a tile is 16 units; TOKENS rows are 128 fp8 bytes
// (16 consecutive tokens of one page: 2 KB contiguous), BLOCKS rows are 256
// bytes of bf16 (one summary row per block, scattered by the page table).
//
// TOKENS tiles go straight from memory into the MFMA B operand: lane
// (col, kq) loads bytes [16 kq, +16) and [64 + 16 kq, +16) of unit col's row
// (each instruction reads the 16 rows' first or second halves), and k-step s
// takes dims 16 kq + 8 s (s < 2) or 64 + 16 kq + 8 (s - 2) (s >= 2). The q
// operand uses the same dims, which leaves every dot product unchanged.
// BLOCKS tiles are loaded row-major and transposed through LDS.
template <int MODE>
struct IdxTile {
  static constexpr int kRowBytes = MODE == kIdxTokens ? kIdxDim : 2 * kIdxDim;
  static constexpr int NL = 16 * kRowBytes / (kWave * 16);   // 16-byte loads per lane
  static constexpr int RPI = kWave * 16 / kRowBytes;         // rows per load instruction
  static constexpr int LPR = kRowBytes / 16;                 // lanes per row
  static constexpr int RW = kRowBytes / 4 + 4;               // LDS row stride (words), padded
};

// Dim of element e (0..7) of k-step s in lane group kq (the q operand's
// layout; see above).
template <int MODE>
__device__ __forceinline__ int idx_kstep_dim(int s, int kq) {
  if constexpr (MODE == kIdxTokens) return s < 2 ? 16 * kq + 8 * s : 64 + 16 * kq + 8 * (s - 2);
  else return 32 * kq + 8 * s;
}

template <int MODE, int NHT>
struct IdxScoreLds {
  alignas(16) uint32_t tiles[MODE == kIdxTokens ? 1 : kIdxWaves][2][16 * IdxTile<MODE>::RW];
  uint4 q[NHT][4][kWave];   // the q operand, in lane order (one 16-byte read per lane)
  // page ids of the workgroup's blocks (one per 16+ tokens, one per block),
  // or with token candidates the key row of every unit
  int pg[kIdxMaxTilesPerWg * 16];
  // token mode, block units: cached tokens of each of those blocks (a unit
  // is valid when its slot is below this; 0 for a block that is not scored)
  int nv[kIdxMaxTilesPerWg * 16 / 16 + 1];
  float red[2 * kIdxWaves];
};

template <int MODE, int NHT>
__global__ __launch_bounds__(kIdxThreads, 2) void idx_score_kernel(IndexerArgs a) {
  using T = IdxTile<MODE>;
  constexpr int NL = T::NL, NS = kIdxPrefetch, H = 16 * NHT;
  static_assert(MODE != kIdxTokens || NL == 2, "token rows: two 16-byte loads per lane");
  __shared__ IdxScoreLds<MODE, NHT> sh;
  const int r = blockIdx.y, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int P = a.b.page_size;                 // 16, 32 or 64
  const int PS = __builtin_ctz((unsigned)P);    // units -> (block, slot) by shift and mask
  const int upw = a.tiles_per_wg * 16;
  const int u0 = blockIdx.x * upw;

  // the request's units
  int n_units, c0 = 0, c1 = 0;
  IdxUnits gu;
  if constexpr (MODE == kIdxTokens) {
    gu = idx_units(a, r);
    n_units = gu.n;
  } else {
    const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
    n_units = geo.nb;
    c0 = geo.c0;
    c1 = geo.c1;
    gu.page_base = geo.page_base;
    gu.nb = geo.nb;
  }
  if (MODE == kIdxTokens && blockIdx.x == 0) idx_clear_request<kIdxThreads>(a, r);
  if (u0 >= n_units) return;

  // page ids of the workgroup's blocks (-1: no unit of this block is scored)
  const int bi0 = MODE == kIdxTokens ? u0 >> PS : u0;
  const int npg = MODE == kIdxTokens ? (upw + P - 1) >> PS : upw;
  const bool tok_cands = MODE == kIdxTokens && a.unit_kind == kUnitsTokenCands;
  if (tok_cands) {
    // key row (page * P + slot) of each unit: -1 not a token, -2 bad page;
    // every thread's loads issued before the dependent ones
    constexpr int NPT = kIdxMaxTilesPerWg * 16 / kIdxThreads;
    int tok[NPT], blk[NPT], pgid[NPT];
#pragma unroll
    for (int m = 0; m < NPT; ++m) {
      const int i = tid + m * kIdxThreads;
      blk[m] = i < upw ? idx_unit_block(a, gu, r, u0 + i, &tok[m]) : -1;
    }
#pragma unroll
    for (int m = 0; m < NPT; ++m) pgid[m] = blk[m] >= 0 ? a.b.indices[gu.page_base + blk[m]] : -1;
#pragma unroll
    for (int m = 0; m < NPT; ++m) {
      const int i = tid + m * kIdxThreads;
      if (i < upw)
        sh.pg[i] = blk[m] < 0 ? -1
                 : (pgid[m] >= 0 && pgid[m] < a.b.num_pages) ? pgid[m] * P + (tok[m] & (P - 1))
                                                              : -2;
    }
  }
  for (int i = tid; i < npg && !tok_cands; i += kIdxThreads) {
    const int bi = bi0 + i;
    int page = -1;
    if constexpr (MODE == kIdxTokens) {
      int blk = -1;
      if (gu.ncand < 0) blk = bi < gu.nb ? bi : -1;
      else if (bi < gu.ncand) blk = a.cand_blocks[(size_t)r * a.cand_cap + bi];
      int nvt = 0;
      if (blk >= 0 && blk < gu.nb) {
        const int p = a.b.indices[gu.page_base + blk];
        page = (p >= 0 && p < a.b.num_pages) ? p : -2;   // -2: bad page id, scores 0
        nvt = gu.L - blk * P;
        nvt = nvt < 0 ? 0 : (nvt > P ? P : nvt);
      }
      sh.nv[i] = nvt;
    } else {
      if (bi >= c0 && bi < c1) {
        const int p = a.b.indices[gu.page_base + bi];
        page = (p >= 0 && p < a.b.num_pages) ? p : -2;
      }
    }
    sh.pg[i] = page;
  }

  // q (A operand: row = head 16ht + col, dims 32kq + 8s .. +8 of k-step s),
  // loaded once per workgroup through LDS and then held in registers (read
  // from LDS per tile it cost 16 KB of LDS reads per wave and tile, which
  // bounded the loop), and the head weights of this lane's output rows
  // (heads 16ht + 4kq + i)
  float wv[NHT][4];
  {
    constexpr int NQ = NHT * 4 * kWave / kIdxThreads;   // every load issued before the stores
    uint4 qv[NQ];
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int e = tid + m * kIdxThreads;
      const int ht = e / (4 * kWave), s = (e / kWave) % 4, ln = e % kWave;
      qv[m] = ldg16(a.q + ((size_t)r * H + 16 * ht + (ln & 15)) * kIdxDim +
                    idx_kstep_dim<MODE>(s, ln >> 4));
    }
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      const int e = tid + m * kIdxThreads;
      sh.q[e / (4 * kWave)][(e / kWave) % 4][e % kWave] = qv[m];
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
    for (int s2 = 0; s2 < 4; ++s2) qr[ht][s2] = sh.q[ht][s2][lane];

  const int ntw = a.tiles_per_wg / kIdxWaves;
  float* srow = a.scores + (size_t)r * a.max_units + u0;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys);
  // the row this lane loads with instruction j of the wave's k-th tile and
  // its page slot (-1: not scored, -2: bad page)
  auto row_page = [&](int k, int j, size_t* off) {
    const int t = wave + kIdxWaves * k;           // tile in the workgroup
    const int u = 16 * t + j * T::RPI + lane / T::LPR;   // unit of the row (in the wg)
    int pslot, page;
    if constexpr (MODE == kIdxTokens) {
      pslot = ((u0 + u) >> PS) - bi0;
      page = k < ntw ? sh.pg[pslot] : -1;
      const int slot = (u0 + u) & (P - 1);
      *off = ((size_t)(uint32_t)(page >= 0 ? page : 0) * P + slot) * kIdxDim;
    } else {
      pslot = u;
      page = k < ntw ? sh.pg[pslot] : -1;
      *off = (size_t)(uint32_t)(page >= 0 ? page : 0) * (2 * kIdxDim);
    }
    return page;
  };
  auto issue = [&](int k, uint4* d, uint32_t& badm, float& sig) {
    badm = 0;
    if constexpr (MODE == kIdxTokens) {
      // this lane's own unit (col) of the wave's k-th tile, both halves
      const int ul = 16 * (wave + kIdxWaves * k) + col, u = u0 + ul;
      size_t row;
      if (tok_cands) {
        const int kr = k < ntw ? sh.pg[ul] : -1;
        badm = kr == -2 ? 0x3u : 0u;
        row = (size_t)(uint32_t)(kr >= 0 ? kr : 0);
      } else {
        const int page = k < ntw ? sh.pg[(u >> PS) - bi0] : -1;
        badm = page == -2 ? 0x3u : 0u;
        row = (size_t)(uint32_t)(page >= 0 ? page : 0) * P + (u & (P - 1));
      }
      const uint8_t* rowp = kbase + (size_t)row * kIdxDim;
      d[0] = ldg16_stream(rowp + 16 * kq);
      d[1] = ldg16_stream(rowp + 64 + 16 * kq);
      sig = a.scales ? a.scales[row] : 1.0f;
    } else {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        size_t off;
        const int page = row_page(k, j, &off);
        badm |= (uint32_t)(page == -2) << j;
        d[j] = ldg16(kbase + off + 16 * (lane % T::LPR));
      }
    }
    if constexpr (MODE != kIdxTokens) sig = 1.0f;
  };

  uint4 buf[NS][NL];
  uint32_t badm[NS];
  float sig[NS];
  float rmn = __builtin_inff(), rmx = -__builtin_inff();   // range of this thread's valid scores
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    issue(s, buf[s], badm[s], sig[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int k0 = 0; k0 < ntw; k0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int k = k0 + s;
      uint4 c[NL];
      const uint32_t bm = badm[s];
      const float sg = sig[s];
#pragma unroll
      for (int j = 0; j < NL; ++j) c[j] = buf[s][j];
      __builtin_amdgcn_sched_barrier(0);
      issue(k + NS, buf[s], badm[s], sig[s]);
      __builtin_amdgcn_sched_barrier(0);
      if (k < ntw) {
        // B operand (key^T): unit `col`, the dims idx_kstep_dim gives
        uint4 kb[4];
        if constexpr (MODE == kIdxTokens) {
          // a unit with a bad page scores 0 (its bytes are replaced by zeros;
          // the wave-wide test keeps the common case free of per-lane selects)
          uint4 x0 = c[0], x1 = c[1];
          if (__ballot(bm != 0u) != 0) {
            if (bm) {
              x0 = make_uint4(0, 0, 0, 0);
              x1 = make_uint4(0, 0, 0, 0);
            }
          }
          const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            kb[s2] = make_uint4(fp8x2_to_bf16x2(xs[2 * s2], false),
                                fp8x2_to_bf16x2(xs[2 * s2], true),
                                fp8x2_to_bf16x2(xs[2 * s2 + 1], false),
                                fp8x2_to_bf16x2(xs[2 * s2 + 1], true));
        } else {
          uint32_t* tile = sh.tiles[wave][s & 1];
          // stage row-major (rows with a bad page become zeros)
#pragma unroll
          for (int j = 0; j < NL; ++j) {
            const int row = j * T::RPI + lane / T::LPR;
            *reinterpret_cast<uint4*>(tile + row * T::RW + 4 * (lane % T::LPR)) =
                ((bm >> j) & 1u) ? make_uint4(0, 0, 0, 0) : c[j];
          }
          wave_lds_sync();
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            kb[s2] = *reinterpret_cast<const uint4*>(tile + col * T::RW + 16 * kq + 4 * s2);
        }
        // k-step outer, head tile inner: the NHT products of a k-step are
        // independent, so the matrix core is not left waiting on a result
        f32x4_t acc[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) acc[ht] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) acc[ht] = mfma_16x16x32(qr[ht][s2], kb[s2], acc[ht]);
        // s = sum_h w_h max(0, sigma * d_h); lane holds heads 16ht + 4kq + i
        float v = 0.0f;
        if (__ballot(!(sg > 0.0f)) == 0) {   // all scales positive: sigma factors out
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) v = fmaf(wv[ht][i], relu_bits(acc[ht][i]), v);
          v = xor_pair_sum<16>(v);
          v = xor_pair_sum<32>(v);
          v *= sg;
        } else {
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) v = fmaf(wv[ht][i], relu_bits(acc[ht][i] * sg), v);
          v = xor_pair_sum<16>(v);
          v = xor_pair_sum<32>(v);
        }
        v += 0.0f;   // -0 -> +0: equal scores get equal keys
        if (kq == 0) {
          const int t = wave + kIdxWaves * k;
          const int ul = 16 * t + col;   // unit in the workgroup
          bool valid;
          if constexpr (MODE == kIdxTokens) {
            // from LDS: a memory read here would make the wait for it also
            // wait for the key tiles in flight
            const int uu = u0 + ul;
            valid = tok_cands ? sh.pg[ul] != -1 : (uu & (P - 1)) < sh.nv[(uu >> PS) - bi0];
            if (valid) {
              rmn = fminf(rmn, v);
              rmx = fmaxf(rmx, v);
            }
          } else {
            valid = u0 + ul >= c0 && u0 + ul < c1;
          }
          if (u0 + ul < n_units) srow[ul] = valid ? v : 0.0f;
        }
      }
    }
  }
  if constexpr (MODE == kIdxTokens) {
    idx_range_reduce<kIdxThreads>(rmn, rmx, sh.red);
    if (tid == 0)
      a.range[(size_t)r * (a.max_units / kIdxMinWgUnits) + blockIdx.x] = make_float2(rmn, rmx);
  }
}

// ------------------------------------------------------------ token top-k ----

constexpr int kIdxMarkThreads = 512;
constexpr int kIdxMarkWaves = kIdxMarkThreads / kWave;

struct IdxMarkLds {
  alignas(16) uint32_t h[kIdxBins];   // digit histograms; the finish also lists units here
  uint32_t h2[kIdxBins];       // finish: the candidate blocks (unit -> token map)
  uint32_t bm[kIdxMaxWords];   // finish: selected units
  uint32_t tie[kIdxMaxWords];  // finish: units equal to the k-th key
  int red[kIdxMarkWaves];
  int bstar, cabove, kr, last, dig, above;
};

// Exclusive prefix sum over the workgroup in thread order; *total = sum.
__device__ __forceinline__ int idx_block_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kIdxMarkWaves; ++w) {
    const int x = red[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// Digit search from the top over h[0 .. nbins) (a power of two, 16 ..
// kIdxBins): the bin b with (count above b) < need <= (count at or above b).
// Writes b and the count above it (one thread), then synchronises.
// need >= 1 and sum(h) >= need.
__device__ __forceinline__ void idx_find_digit(const uint32_t* h, int nbins, int need, int* red,
                                               int* b_out, int* above_out) {
  const int per = nbins > kIdxMarkThreads ? nbins / kIdxMarkThreads : 1;
  const int t = threadIdx.x, own = t * per < nbins;
  int mine = 0;
  if (own)
    for (int i = 0; i < per; ++i) mine += (int)h[t * per + i];
  int tot;
  const int excl = idx_block_scan(mine, red, &tot);
  int above = tot - excl - mine;   // elements in bins of higher threads
  if (own && above < need && above + mine >= need) {
    for (int b = t * per + per - 1; b >= t * per; --b) {
      if (above + (int)h[b] >= need) {
        *b_out = b;
        *above_out = above;
        break;
      }
      above += (int)h[b];
    }
  }
  __syncthreads();
}

// dst[i] = src[i] for i < n (n <= NPT * kIdxMarkThreads), every load of a
// thread issued before its stores (a plain strided loop would wait out one
// memory round trip per iteration). kDev: device-coherent loads, for words
// that other workgroups of the same launch wrote.
template <int NPT, bool kDev = false>
__device__ __forceinline__ void idx_copy_in(uint32_t* dst, const uint32_t* src, int n) {
  uint32_t v[NPT];
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int i = threadIdx.x + m * kIdxMarkThreads;
    v[m] = i < n ? ld_x<kDev>(src + i) : 0u;
  }
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int i = threadIdx.x + m * kIdxMarkThreads;
    if (i < n) dst[i] = v[m];
  }
}

// A listed unit (score bits, unit) written by another workgroup of the same
// launch, read device-coherently.
__device__ __forceinline__ uint2 ld_dev_u2(const uint2* p) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
  return make_uint2(ld_dev(w), ld_dev(w + 1));
}

__device__ __forceinline__ int idx_token_of(const IndexerArgs& a, const IdxUnits& g, int r,
                                           int u) {
  if (a.unit_kind == kUnitsTokenCands)
    return u < g.ncand ? a.cand_blocks[(size_t)r * a.cand_cap + u] : g.tail0 + (u - g.ncand);
  if (g.ncand < 0) return u;
  const int P = a.b.page_size, PS = __builtin_ctz((unsigned)P);
  return a.cand_blocks[(size_t)r * a.cand_cap + (u >> PS)] * P + (u & (P - 1));
}

// The request's remap (min and scale, as float bits in ctl[2], ctl[3]) from
// the scoring workgroups' range slots, and the histogram of the first digit
// (bucket >> 4) of this chunk's valid units. One workgroup per
// (kIdxMarkUnits units, request).
constexpr int kIdxHistThreads = 256;
__global__ __launch_bounds__(kIdxHistThreads) void idx_hist_kernel(IndexerArgs a) {
  __shared__ uint32_t h[kIdxCoarse];
  __shared__ float red[2 * kIdxHistThreads / kWave];
  const int r = blockIdx.y, tid = threadIdx.x;
  const IdxUnits g = idx_units(a, r);
  const int cu0 = blockIdx.x * kIdxMarkUnits;
  if (cu0 >= g.n) return;
  const int upw = a.tiles_per_wg * 16;
  const int nwg = (g.n + upw - 1) / upw;   // the scoring workgroups that wrote a slot
  const float2* slots = a.range + (size_t)r * (a.max_units / kIdxMinWgUnits);
  float mn = __builtin_inff(), mx = -__builtin_inff();
  for (int i = tid; i < nwg; i += kIdxHistThreads) {
    const float2 m = slots[i];
    mn = fminf(mn, m.x);
    mx = fmaxf(mx, m.y);
  }
  for (int i = tid; i < kIdxCoarse; i += kIdxHistThreads) h[i] = 0u;
  idx_range_reduce<kIdxHistThreads>(mn, mx, red);
  const float scale = idx_remap_scale(mn, mx);
  if (blockIdx.x == 0 && tid == 0) {
    a.ctl[(size_t)r * 4 + 2] = __float_as_uint(mn);
    a.ctl[(size_t)r * 4 + 3] = __float_as_uint(scale);
  }
  constexpr int IT = kIdxMarkUnits / kIdxHistThreads;
  const float* srow = a.scores + (size_t)r * a.max_units;
  float sv[IT];
  bool vv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {   // every score load in flight at once
    const int u = cu0 + it * kIdxHistThreads + tid;
    int tok;
    vv[it] = idx_unit_block(a, g, r, u, &tok) >= 0;
    sv[it] = vv[it] ? srow[u] : 0.0f;
  }
#pragma unroll
  for (int it = 0; it < IT; ++it)
    if (vv[it]) atomicAdd(&h[idx_remap_bin(sv[it], mn, scale) >> 4], 1u);
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)r * kIdxCoarse;
  for (int i = tid; i < kIdxCoarse; i += kIdxHistThreads) {
    const uint32_t c = h[i];
    if (c) atomicAdd(gh + i, c);
  }
}

__global__ __launch_bounds__(kIdxMarkThreads) void idx_mark_kernel(IndexerArgs a) {
  __shared__ IdxMarkLds sh;
  const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const IdxUnits g = idx_units(a, r);
  const int nwords_row = a.max_units / 32;
  uint32_t* bmrow = a.bitmap + (size_t)r * nwords_row;
  uint32_t* ctl = a.ctl + (size_t)r * 4;
  const float* srow = a.scores + (size_t)r * a.max_units;
  uint2* crow = a.cand + (size_t)r * a.max_units;
  const float rmn = __uint_as_float(ctl[2]), rscale = __uint_as_float(ctl[3]);

  // 1. the first digit d* holding the k-th score, from the request's histogram
  const uint32_t* gh = a.hist + (size_t)r * kIdxCoarse;
  idx_copy_in<1>(sh.h, gh, kIdxCoarse);
  if (tid == 0) {
    sh.bstar = kIdxCoarse;   // nothing definite, no candidates
    sh.cabove = 0;
  }
  __syncthreads();
  {
    const int mine = tid < kIdxCoarse ? (int)sh.h[tid] : 0;
    int tot;
    const int excl = idx_block_scan(mine, sh.red, &tot);
    const int kr = a.topk < tot ? a.topk : tot;
    if (tid == 0) {
      sh.kr = kr;
      if (kr >= tot && tot > 0) sh.bstar = -1;   // every valid unit is selected
    }
    const int above = tot - excl - mine;   // units in higher digits
    if (kr > 0 && kr < tot && tid < kIdxCoarse && above < kr && above + mine >= kr) {
      sh.bstar = tid;
      sh.cabove = above;
    }
  }
  __syncthreads();
  const int bstar = sh.bstar;
  const bool refine = bstar >= 0 && bstar < kIdxCoarse;

  // 2. this chunk: selected bits above d*; units of d* to the candidate list
  const int cu0 = chunk * kIdxMarkUnits;
  constexpr int IT = kIdxMarkUnits / kIdxMarkThreads;
  float sv[IT];
  bool vv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {   // all of this thread's score loads in flight at once
    const int u = cu0 + it * kIdxMarkThreads + wave * kWave + lane;
    int tok;
    vv[it] = idx_unit_block(a, g, r, u, &tok) >= 0;
    sv[it] = vv[it] ? srow[u] : 0.0f;
  }
  // selected bits; this wave's digit-d* units counted first, so that the
  // workgroup reserves its slots of the list with ONE returning atomic
  unsigned long long cmask[IT];
  int wcount = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int ub = cu0 + it * kIdxMarkThreads + wave * kWave;   // wave's 64 units
    const bool valid = vv[it];
    const int bin = idx_remap_bin(sv[it], rmn, rscale) >> 4;   // first digit
    const bool def = valid && (bstar < 0 || bin > bstar);
    cmask[it] = __ballot(refine && valid && bin == bstar);
    wcount += __popcll(cmask[it]);
    const unsigned long long dm = __ballot(def);
    if (lane == 0 && ub < g.n) {
      st_dev(bmrow + ub / 32, (uint32_t)dm);
      st_dev(bmrow + ub / 32 + 1, (uint32_t)(dm >> 32));
    }
  }
  if (lane == 0) sh.red[wave] = wcount;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kIdxMarkWaves; ++w) {
      const int c = sh.red[w];
      sh.red[w] = tot;   // the wave's offset in the workgroup's slots
      tot += c;
    }
    sh.dig = tot ? (int)atomicAdd(ctl, (uint32_t)tot) : 0;   // the workgroup's first slot
  }
  __syncthreads();
  int cpos = sh.dig + sh.red[wave];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const unsigned long long cm = cmask[it];
    if (cm) {
      if ((cm >> lane) & 1ull) {
        const int u = cu0 + it * kIdxMarkThreads + wave * kWave + lane;
        st_dev(crow + cpos + mbcnt(cm), make_uint2(__float_as_uint(sv[it]), (uint32_t)u));
      }
      cpos += __popcll(cm);
    }
  }
  // 3. arrival; the last workgroup of the request finishes it. Everything
  // handed over (bitmap words, listed units, the list counter) goes through
  // device-coherent stores or atomics, which write through the XCD's L2,
  // and every thread waits for its own to complete before the workgroup's
  // arrival is counted (no release fence: that would write back the whole
  // L2 under every other workgroup). The finishing workgroup reads every
  // handed-over word with device-coherent loads (ld_dev), issued after its
  // arrival atomic has returned, so it needs no acquire fence (whose L2
  // invalidation cost about 3 us here); what earlier launches wrote (the
  // candidate blocks) is read with plain loads.
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ctl + 1, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh.last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!sh.last) return;

  const int kr = sh.kr;
  const int nwr = (g.n + 31) / 32;
  idx_copy_in<kIdxMaxWords / kIdxMarkThreads, true>(sh.bm, bmrow, nwr);
  for (int w = tid; w < nwr; w += kIdxMarkThreads) sh.tie[w] = 0u;
  // the candidate blocks (unit -> token map), in LDS when they fit
  const bool cand_lds = a.unit_kind == kUnitsDefault && g.ncand >= 0 && g.ncand <= kIdxBins;
  if (cand_lds)
    idx_copy_in<kIdxBins / kIdxMarkThreads>(
        sh.h2, reinterpret_cast<const uint32_t*>(a.cand_blocks + (size_t)r * a.cand_cap), g.ncand);
  int ties_to_take = 0;
  constexpr int UN = 4;   // candidate loads in flight per thread
  const int nc = refine ? (int)ld_dev(ctl) : 0;   // units with digit d*
  const bool approx = a.approx == 1;
  // what ranks a listed unit (larger first): its key, or its bucket for the
  // approximate top-k (the bucket holding the k-th score is then filled in
  // ascending unit order: ties go to the lower unit)
  auto rank_key = [&](uint32_t sbits) -> uint32_t {
    const float sc = __uint_as_float(sbits);
    return approx ? (uint32_t)idx_remap_bin(sc, rmn, rscale) : score_key(sc);
  };
  // one pass over the listed units: f(rank key, unit) for each
  auto each_listed = [&](auto&& f) {
    for (int i0 = 0; i0 < nc; i0 += UN * kIdxMarkThreads) {
      uint2 c[UN];
#pragma unroll
      for (int j = 0; j < UN; ++j) {
        const int i = i0 + j * kIdxMarkThreads + tid;
        c[j] = i < nc ? ld_dev_u2(crow + i) : make_uint2(0u, 0xFFFFFFFFu);
      }
#pragma unroll
      for (int j = 0; j < UN; ++j)
        if (c[j].y != 0xFFFFFFFFu) f(rank_key(c[j].x), c[j].y);
    }
  };
  int need = kr - sh.cabove;   // units of digit d* to select (>= 1 when refining)
  if (refine && nc <= kIdxMarkThreads) {
    // few listed units (the remap's purpose): each thread ranks one of them
    // against all, by (rank key descending, unit ascending), in LDS
    // as one 64-bit key (rank key << 32 | ~unit): a unit's rank is the number
    // of larger keys. The list is padded to a multiple of 16 entries with key
    // 0, which is larger than nothing, and read 16 bytes at a time, 8 reads
    // in flight.
    unsigned long long* lst = reinterpret_cast<unsigned long long*>(sh.h);   // <= 512: 4 KB of h
    const int ncp = (nc + 15) & ~15;
    unsigned long long me = 0ull;
    if (tid < nc) {
      const uint2 c = ld_dev_u2(crow + tid);
      me = ((unsigned long long)rank_key(c.x) << 32) | (uint32_t)~c.y;
    }
    if (tid < ncp) lst[tid] = me;
    __syncthreads();
    if (tid < nc) {
      const ulonglong2* l2 = reinterpret_cast<const ulonglong2*>(lst);
      int rank = 0;
      for (int j = 0; j < ncp / 2; j += 8) {
        ulonglong2 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = l2[j + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) rank += (int)(v[q].x > me) + (int)(v[q].y > me);
      }
      const uint32_t u = ~(uint32_t)me;
      if (rank < need) atomicOr(&sh.bm[u >> 5], 1u << (u & 31));
    }
  } else if (refine) {
    // digits of the rank key among the listed units: [31:20], [19:8], [7:0]
    // (a bucket has 12 bits: its second and third digits are 0), each among
    // the units that share the digits found so far
    uint32_t prefix = 0u, pmask = 0u;
    for (int d = 0; d < 3; ++d) {
      const int shift = d == 0 ? 20 : (d == 1 ? 8 : 0);
      const int nbins = d == 2 ? 256 : kIdxBins;
      for (int i = tid; i < nbins; i += kIdxMarkThreads) sh.h[i] = 0u;
      __syncthreads();
      each_listed([&](uint32_t key, uint32_t) {
        if ((key & pmask) == prefix) atomicAdd(&sh.h[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
      });
      __syncthreads();
      idx_find_digit(sh.h, nbins, need, sh.red, &sh.dig, &sh.above);
      prefix |= (uint32_t)sh.dig << shift;
      pmask |= (uint32_t)(nbins - 1) << shift;
      need -= sh.above;
      __syncthreads();   // dig / above are rewritten by the next digit
    }
    const uint32_t theta = prefix;   // the k-th rank key
    ties_to_take = need;
    each_listed([&](uint32_t key, uint32_t u) {
      if (key > theta) atomicOr(&sh.bm[u >> 5], 1u << (u & 31));
      else if (key == theta) atomicOr(&sh.tie[u >> 5], 1u << (u & 31));
    });
  }
  __syncthreads();

  // 4. emit in ascending unit order: the bitmap plus the first ties. Thread
  // t owns words [t wpt, (t + 1) wpt), held in registers (wpt <= 16).
  const int P = a.b.page_size, PS = __builtin_ctz((unsigned)P);
  constexpr int WMAX = kIdxMaxWords / kIdxMarkThreads;
  const int wpt = (nwr + kIdxMarkThreads - 1) / kIdxMarkThreads;
  const int w0 = tid * wpt;
  uint32_t bw[WMAX];
#pragma unroll
  for (int i = 0; i < WMAX; ++i) bw[i] = (i < wpt && w0 + i < nwr) ? sh.bm[w0 + i] : 0u;
  if (ties_to_take > 0) {   // uniform: the first ties_to_take tie units join
    uint32_t tw[WMAX];
    int tcount = 0;
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      tw[i] = (i < wpt && w0 + i < nwr) ? sh.tie[w0 + i] : 0u;
      tcount += __popc(tw[i]);
    }
    int ttot;
    int tpre = idx_block_scan(tcount, sh.red, &ttot);
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      uint32_t x = tw[i], kept = 0u;
      const int pc = __popc(x);
      int take = ties_to_take - tpre;
      take = take < 0 ? 0 : (take > pc ? pc : take);
      for (int j = 0; j < take; ++j) {
        const uint32_t low = x & (0u - x);
        kept |= low;
        x ^= low;
      }
      tpre += pc;
      bw[i] |= kept;
    }
  }
  int scount = 0;
#pragma unroll
  for (int i = 0; i < WMAX; ++i) scount += __popc(bw[i]);
  int stot;
  int pos = idx_block_scan(scount, sh.red, &stot);
  int32_t* out = a.selected + (size_t)r * a.max_selected;
  // one loop per unit -> token map: a map that reads global memory (token
  // candidates) would make every store of a shared loop wait for all memory
  // operations before it, the earlier stores included
  auto emit_all = [&](auto token_of) {
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      uint32_t x = bw[i];
      while (x) {
        const int b = __ffs(x) - 1;
        x &= x - 1u;
        if (pos < a.max_selected) out[pos] = token_of(32 * (w0 + i) + b);
        ++pos;
      }
    }
  };
  if (cand_lds)
    emit_all([&](int u) { return (int)sh.h2[u >> PS] * P + (u & (P - 1)); });
  else if (a.unit_kind != kUnitsTokenCands && g.ncand < 0)
    emit_all([](int u) { return u; });
  else
    emit_all([&](int u) { return idx_token_of(a, g, r, u); });
  for (int i = stot + tid; i < a.max_selected; i += kIdxMarkThreads) out[i] = -1;
  if (tid == 0) a.selected_count[r] = stot < a.max_selected ? stot : a.max_selected;
}

// -------------------------------------------------------------- launch ----

template <int MODE>
static hipError_t launch_score_mode(const IndexerArgs& a, hipStream_t st) {
  const int upw = a.tiles_per_wg * 16;
  dim3 grid((a.max_units + upw - 1) / upw, a.b.batch);
  switch (a.num_heads) {
    case 16: hipLaunchKernelGGL((idx_score_kernel<MODE, 1>), grid, dim3(kIdxThreads), 0, st, a); break;
    case 32: hipLaunchKernelGGL((idx_score_kernel<MODE, 2>), grid, dim3(kIdxThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((idx_score_kernel<MODE, 4>), grid, dim3(kIdxThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_indexer_score(const IndexerArgs& a, int mode, hipStream_t st) {
  return mode == kIdxTokens ? launch_score_mode<kIdxTokens>(a, st)
                            : launch_score_mode<kIdxBlocks>(a, st);
}

hipError_t launch_indexer_hist(const IndexerArgs& a, hipStream_t st) {
  dim3 grid((a.max_units + kIdxMarkUnits - 1) / kIdxMarkUnits, a.b.batch);
  hipLaunchKernelGGL(idx_hist_kernel, grid, dim3(kIdxHistThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_indexer_mark(const IndexerArgs& a, hipStream_t st) {
  dim3 grid((a.max_units + kIdxMarkUnits - 1) / kIdxMarkUnits, a.b.batch);
  hipLaunchKernelGGL(idx_mark_kernel, grid, dim3(kIdxMarkThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_indexer_token_select(const IndexerArgs& a, hipStream_t st) {
  hipError_t e = launch_score_mode<kIdxTokens>(a, st);
  if (e != hipSuccess) return e;
  e = launch_indexer_hist(a, st);
  if (e != hipSuccess) return e;
  return launch_indexer_mark(a, st);
}

}  // namespace ls

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
  uint32_t hist[MODE == kIdxTokens ? kIdxBins : 1];
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
      if (blk >= 0 && blk < gu.nb) {
        const int p = a.b.indices[gu.page_base + blk];
        page = (p >= 0 && p < a.b.num_pages) ? p : -2;   // -2: bad page id, scores 0
      }
    } else {
      if (bi >= c0 && bi < c1) {
        const int p = a.b.indices[gu.page_base + bi];
        page = (p >= 0 && p < a.b.num_pages) ? p : -2;
      }
    }
    sh.pg[i] = page;
  }
  if constexpr (MODE == kIdxTokens) {
    for (int i = tid; i < kIdxBins; i += kIdxThreads) sh.hist[i] = 0u;
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
        f32x4_t acc[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          acc[ht] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) acc[ht] = mfma_16x16x32(qr[ht][s2], kb[s2], acc[ht]);
        }
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
            int tok;
            valid = idx_unit_block(a, gu, r, u0 + ul, &tok) >= 0;
            if (valid) atomicAdd(&sh.hist[idx_bin(score_key(v))], 1u);
          } else {
            valid = u0 + ul >= c0 && u0 + ul < c1;
          }
          if (u0 + ul < n_units) srow[ul] = valid ? v : 0.0f;
        }
      }
    }
  }
  __syncthreads();
  if constexpr (MODE == kIdxTokens) {
    uint32_t* gh = a.hist + (size_t)r * kIdxBins;
    for (int i = tid; i < kIdxBins; i += kIdxThreads) {
      const uint32_t c = sh.hist[i];
      if (c) atomicAdd(gh + i, c);
    }
  }
}

// ------------------------------------------------------------ token top-k ----

// One 16-byte store per thread (the histograms are 256-byte aligned).
__global__ __launch_bounds__(kIdxThreads) void idx_zero_kernel(uint32_t* hist, uint32_t* ctl,
                                                               int batch) {
  const int n4 = 2 * batch * kIdxBins / 4;   // first-digit and second-digit histograms
  const int i = blockIdx.x * kIdxThreads + threadIdx.x;
  if (i < n4) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (i < batch * 4) ctl[i] = 0u;
}

constexpr int kIdxMarkThreads = 512;
constexpr int kIdxMarkWaves = kIdxMarkThreads / kWave;

struct IdxMarkLds {
  uint32_t h[kIdxBins];        // digit histograms (first, then second, then third digit)
  uint32_t h2[kIdxBins];       // this workgroup's second-digit histogram of bucket b*
  uint32_t bm[kIdxMaxWords];   // finish: selected units
  uint32_t tie[kIdxMaxWords];  // finish: units equal to the k-th key
  int red[kIdxMarkWaves];
  int bstar, cabove, kr, last, b2, above2, b3, above3;
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

// Digit search from the top over h[0 .. nbins) (nbins a multiple of the
// workgroup size): the bin b with (count above b) < need <= (count at or
// above b). Writes b and the count above it (one thread), then synchronises.
// need >= 1 and sum(h) >= need.
__device__ __forceinline__ void idx_find_digit(const uint32_t* h, int nbins, int need, int* red,
                                               int* b_out, int* above_out) {
  const int per = nbins / kIdxMarkThreads, t = threadIdx.x;
  int mine = 0;
  for (int i = 0; i < per; ++i) mine += (int)h[t * per + i];
  int tot;
  const int excl = idx_block_scan(mine, red, &tot);
  int above = tot - excl - mine;   // elements in bins of higher threads
  if (above < need && above + mine >= need) {
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

__device__ __forceinline__ int idx_token_of(const IndexerArgs& a, const IdxUnits& g, int r,
                                           int u) {
  if (a.unit_kind == kUnitsTokenCands)
    return u < g.ncand ? a.cand_blocks[(size_t)r * a.cand_cap + u] : g.tail0 + (u - g.ncand);
  if (g.ncand < 0) return u;
  const int P = a.b.page_size, PS = __builtin_ctz((unsigned)P);
  return a.cand_blocks[(size_t)r * a.cand_cap + (u >> PS)] * P + (u & (P - 1));
}

// dst[i] = src[i] for i < n (n <= NPT * kIdxMarkThreads), every load of a
// thread issued before its stores (a plain strided loop would wait out one
// memory round trip per iteration).
template <int NPT>
__device__ __forceinline__ void idx_copy_in(uint32_t* dst, const uint32_t* src, int n) {
  uint32_t v[NPT];
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int i = threadIdx.x + m * kIdxMarkThreads;
    v[m] = i < n ? src[i] : 0u;
  }
#pragma unroll
  for (int m = 0; m < NPT; ++m) {
    const int i = threadIdx.x + m * kIdxMarkThreads;
    if (i < n) dst[i] = v[m];
  }
}

// Second digit of a score key: bits [19:8]; third digit: bits [7:0].
__device__ __forceinline__ uint32_t idx_d2(uint32_t key) { return (key >> 8) & 0xFFFu; }

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
  uint32_t* gh2 = a.hist + ((size_t)a.b.batch + r) * kIdxBins;

  // 1. threshold bucket b* from the request's first-digit histogram
  const uint32_t* gh = a.hist + (size_t)r * kIdxBins;
  idx_copy_in<kIdxBins / kIdxMarkThreads>(sh.h, gh, kIdxBins);
  for (int i = tid; i < kIdxBins; i += kIdxMarkThreads) sh.h2[i] = 0u;
  if (tid == 0) {
    sh.bstar = kIdxBins;   // nothing definite, no candidates
    sh.cabove = 0;
  }
  __syncthreads();
  {
    int mine = 0;
    constexpr int per = kIdxBins / kIdxMarkThreads;
    for (int i = 0; i < per; ++i) mine += (int)sh.h[tid * per + i];
    int tot;
    const int excl = idx_block_scan(mine, sh.red, &tot);
    const int kr = a.topk < tot ? a.topk : tot;
    if (tid == 0) {
      sh.kr = kr;
      if (kr >= tot && tot > 0) sh.bstar = -1;   // every valid unit is selected
    }
    if (kr > 0 && kr < tot) {
      int above = tot - excl - mine;
      if (above < kr && above + mine >= kr) {
        for (int b = tid * per + per - 1; b >= tid * per; --b) {
          const int hb = (int)sh.h[b];
          if (above + hb >= kr) {
            sh.bstar = b;
            sh.cabove = above;
            break;
          }
          above += hb;
        }
      }
    }
  }
  __syncthreads();
  const int bstar = sh.bstar;
  const bool refine = bstar >= 0 && bstar < kIdxBins;
  const bool digits = refine && a.approx != 1;   // one-digit approximation: no second digit

  // 2. this chunk: selected bits above b*; units of b* to the candidate list
  // and into the second-digit histogram
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
  // selected bits; this wave's bucket-b* units counted first, so that the
  // workgroup reserves its slots of the list with ONE returning atomic
  uint32_t key[IT];
  unsigned long long cmask[IT];
  int wcount = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int ub = cu0 + it * kIdxMarkThreads + wave * kWave;   // wave's 64 units
    const bool valid = vv[it];
    key[it] = valid ? score_key(sv[it]) : 0u;
    const int bin = (int)idx_bin(key[it]);
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
    sh.b2 = tot ? (int)atomicAdd(ctl, (uint32_t)tot) : 0;   // the workgroup's first slot
  }
  __syncthreads();
  int cpos = sh.b2 + sh.red[wave];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const unsigned long long cm = cmask[it];
    if (cm) {
      if ((cm >> lane) & 1ull) {
        const int u = cu0 + it * kIdxMarkThreads + wave * kWave + lane;
        st_dev(crow + cpos + mbcnt(cm), make_uint2(key[it], (uint32_t)u));
        if (digits) atomicAdd(&sh.h2[idx_d2(key[it])], 1u);
      }
      cpos += __popcll(cm);
    }
  }
  __syncthreads();
  if (digits) {
    for (int i = tid; i < kIdxBins; i += kIdxMarkThreads) {
      const uint32_t c = sh.h2[i];
      if (c) atomicAdd(gh2 + i, c);
    }
  }
  // 3. arrival; the last workgroup of the request finishes it. Everything
  // handed over (bitmap words, listed units, histogram adds, the list
  // counter) goes through device-coherent stores or atomics, which write
  // through the XCD's L2, and every thread waits for its own to complete
  // before the workgroup's arrival is counted (no release fence: that would
  // write back the whole L2 under every other workgroup). The finishing
  // workgroup takes one acquire fence (its XCD's L2 drops stale lines) and
  // then reads everything with plain, pipelined loads.
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ctl + 1, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh.last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!sh.last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const int kr = sh.kr;
  const int nwr = (g.n + 31) / 32;
  idx_copy_in<kIdxMaxWords / kIdxMarkThreads>(sh.bm, bmrow, nwr);
  for (int w = tid; w < nwr; w += kIdxMarkThreads) sh.tie[w] = 0u;
  // the candidate blocks (unit -> token map), in LDS when they fit (h2 is
  // free from here on)
  const bool cand_lds = a.unit_kind == kUnitsDefault && g.ncand >= 0 && g.ncand <= kIdxBins;
  if (cand_lds)
    idx_copy_in<kIdxBins / kIdxMarkThreads>(
        sh.h2, reinterpret_cast<const uint32_t*>(a.cand_blocks + (size_t)r * a.cand_cap), g.ncand);
  int ties_to_take = 0;
  constexpr int UN = 4;   // candidate loads in flight per thread
  if (refine && a.approx == 1) {
    // early exit (Vortex, "Making it fast"): every unit of bucket b* is a
    // tie; the emission takes the first `need` of them in unit order
    const int nc = (int)ld_dev(ctl);
    ties_to_take = kr - sh.cabove;
    __syncthreads();
    for (int i0 = 0; i0 < nc; i0 += UN * kIdxMarkThreads) {
      uint2 c[UN];
#pragma unroll
      for (int j = 0; j < UN; ++j) {
        const int i = i0 + j * kIdxMarkThreads + tid;
        c[j] = i < nc ? crow[i] : make_uint2(0u, 0xFFFFFFFFu);
      }
#pragma unroll
      for (int j = 0; j < UN; ++j)
        if (c[j].y != 0xFFFFFFFFu) atomicOr(&sh.tie[c[j].y >> 5], 1u << (c[j].y & 31));
    }
  } else if (refine) {
    const int need = kr - sh.cabove;   // >= 1 units of bucket b* to select
    const int nc = (int)ld_dev(ctl);   // units in bucket b*
    idx_copy_in<kIdxBins / kIdxMarkThreads>(sh.h, gh2, kIdxBins);
    __syncthreads();
    idx_find_digit(sh.h, kIdxBins, need, sh.red, &sh.b2, &sh.above2);
    const uint32_t b2 = (uint32_t)sh.b2;
    const int need2 = need - sh.above2;
    if (a.approx == 2) {
      // early exit after two digits: units above the 24-bit boundary prefix
      // are selected, the boundary's own units are ties taken in unit order
      const uint32_t theta24 = ((uint32_t)bstar << 12) | b2;
      ties_to_take = need2;
      for (int i0 = 0; i0 < nc; i0 += UN * kIdxMarkThreads) {
        uint2 c[UN];
#pragma unroll
        for (int j = 0; j < UN; ++j) {
          const int i = i0 + j * kIdxMarkThreads + tid;
          c[j] = i < nc ? crow[i] : make_uint2(0u, 0xFFFFFFFFu);
        }
#pragma unroll
        for (int j = 0; j < UN; ++j) {
          if (c[j].y == 0xFFFFFFFFu) continue;
          const uint32_t u = c[j].y, pre = c[j].x >> 8;
          if (pre > theta24) atomicOr(&sh.bm[u >> 5], 1u << (u & 31));
          else if (pre == theta24) atomicOr(&sh.tie[u >> 5], 1u << (u & 31));
        }
      }
    } else {
    // third digit over the candidates whose second digit is b2
    for (int i = tid; i < 256; i += kIdxMarkThreads) sh.h[i] = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < nc; i0 += UN * kIdxMarkThreads) {
      uint2 c[UN];
#pragma unroll
      for (int j = 0; j < UN; ++j) {
        const int i = i0 + j * kIdxMarkThreads + tid;
        c[j] = i < nc ? crow[i] : make_uint2(0u, 0xFFFFFFFFu);
      }
#pragma unroll
      for (int j = 0; j < UN; ++j)
        if (c[j].y != 0xFFFFFFFFu && idx_d2(c[j].x) == b2) atomicAdd(&sh.h[c[j].x & 255u], 1u);
    }
    __syncthreads();
    {
      // 256 bins over 512 threads: the first 256 threads own one bin each
      const int t = tid;
      const int mine = t < 256 ? (int)sh.h[t] : 0;
      int tot;
      const int excl = idx_block_scan(t < 256 ? mine : 0, sh.red, &tot);
      const int above = tot - excl - mine;
      if (t < 256 && above < need2 && above + mine >= need2) {
        sh.b3 = t;
        sh.above3 = above;
      }
      __syncthreads();
    }
    const uint32_t theta = ((uint32_t)bstar << 20) | (b2 << 8) | (uint32_t)sh.b3;
    ties_to_take = need2 - sh.above3;
    for (int i0 = 0; i0 < nc; i0 += UN * kIdxMarkThreads) {
      uint2 c[UN];
#pragma unroll
      for (int j = 0; j < UN; ++j) {
        const int i = i0 + j * kIdxMarkThreads + tid;
        c[j] = i < nc ? crow[i] : make_uint2(0u, 0xFFFFFFFFu);
      }
#pragma unroll
      for (int j = 0; j < UN; ++j) {
        if (c[j].y == 0xFFFFFFFFu) continue;
        const uint32_t u = c[j].y;
        if (c[j].x > theta) atomicOr(&sh.bm[u >> 5], 1u << (u & 31));
        else if (c[j].x == theta) atomicOr(&sh.tie[u >> 5], 1u << (u & 31));
      }
    }
    }
  }
  __syncthreads();

  // 4. emit in ascending unit order: the bitmap plus the first ties
  const int P = a.b.page_size, PS = __builtin_ctz((unsigned)P);
  const int wpt = (nwr + kIdxMarkThreads - 1) / kIdxMarkThreads;
  const int w0 = tid * wpt, w1 = w0 + wpt < nwr ? w0 + wpt : nwr;
  int tcount = 0;
  for (int w = w0; w < w1; ++w) tcount += __popc(sh.tie[w]);
  int ttot;
  int tpre = idx_block_scan(tcount, sh.red, &ttot);
  int scount = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t x = sh.tie[w], kept = 0u;
    int take = ties_to_take - tpre;
    const int pc = __popc(x);
    take = take < 0 ? 0 : (take > pc ? pc : take);
    for (int i = 0; i < take; ++i) {
      const uint32_t low = x & (0u - x);
      kept |= low;
      x ^= low;
    }
    tpre += pc;
    const uint32_t sel = sh.bm[w] | kept;
    sh.bm[w] = sel;
    scount += __popc(sel);
  }
  int stot;
  int pos = idx_block_scan(scount, sh.red, &stot);
  int32_t* out = a.selected + (size_t)r * a.max_selected;
  for (int w = w0; w < w1; ++w) {
    uint32_t x = sh.bm[w];
    while (x) {
      const int b = __ffs(x) - 1;
      x &= x - 1u;
      if (pos < a.max_selected) {
        const int u = 32 * w + b;
        out[pos] = cand_lds ? (int)sh.h2[u >> PS] * P + (u & (P - 1)) : idx_token_of(a, g, r, u);
      }
      ++pos;
    }
  }
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

hipError_t launch_indexer_zero(const IndexerArgs& a, hipStream_t st) {
  const int n4 = 2 * a.b.batch * kIdxBins / 4;
  hipLaunchKernelGGL(idx_zero_kernel, dim3((n4 + kIdxThreads - 1) / kIdxThreads), dim3(kIdxThreads),
                     0, st, a.hist, a.ctl, a.b.batch);
  return hipGetLastError();
}

hipError_t launch_indexer_mark(const IndexerArgs& a, hipStream_t st) {
  dim3 grid((a.max_units + kIdxMarkUnits - 1) / kIdxMarkUnits, a.b.batch);
  hipLaunchKernelGGL(idx_mark_kernel, grid, dim3(kIdxMarkThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_indexer_token_select(const IndexerArgs& a, hipStream_t st) {
  hipError_t e = launch_indexer_zero(a, st);
  if (e != hipSuccess) return e;
  e = launch_score_mode<kIdxTokens>(a, st);
  if (e != hipSuccess) return e;
  return launch_indexer_mark(a, st);
}

}  // namespace ls

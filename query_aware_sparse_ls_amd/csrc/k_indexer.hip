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
template <int MODE>
struct IdxTile {
  static constexpr int kRowBytes = MODE == kIdxTokens ? kIdxDim : 2 * kIdxDim;
  static constexpr int NL = 16 * kRowBytes / (kWave * 16);   // 16-byte loads per lane
  static constexpr int RPI = kWave * 16 / kRowBytes;         // rows per load instruction
  static constexpr int LPR = kRowBytes / 16;                 // lanes per row
  static constexpr int RW = kRowBytes / 4 + 4;               // LDS row stride (words), padded
};

template <int MODE>
struct IdxScoreLds {
  alignas(16) uint32_t tiles[kIdxWaves][2][16 * IdxTile<MODE>::RW];
  float sc[kIdxMaxTilesPerWg * 16];
  int pg[kIdxMaxTilesPerWg * 16 + 1];
  uint32_t hist[MODE == kIdxTokens ? kIdxBins : 1];
};

template <int MODE, int NHT>
__global__ __launch_bounds__(kIdxThreads) void idx_score_kernel(IndexerArgs a) {
  using T = IdxTile<MODE>;
  constexpr int NL = T::NL, NS = kIdxPrefetch, H = 16 * NHT;
  __shared__ IdxScoreLds<MODE> sh;
  const int r = blockIdx.y, tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int P = a.b.page_size;
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
  const int bi0 = MODE == kIdxTokens ? u0 / P : u0;
  const int npg = MODE == kIdxTokens ? (upw + P - 1) / P : upw;
  for (int i = tid; i < npg; i += kIdxThreads) {
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

  // q (A operand: row = head 16ht + col, dims 32kq + 8s .. +8 of k-step s)
  // and the head weights of this lane's output rows (heads 16ht + 4kq + i)
  uint4 qa[NHT][4];
  float wv[NHT][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const uint16_t* qh = a.q + ((size_t)r * H + 16 * ht + col) * kIdxDim + 32 * kq;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[ht][s] = ldg16(qh + 8 * s);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)r * H + 16 * ht + 4 * kq + i];
  }
  __syncthreads();

  const int ntw = a.tiles_per_wg / kIdxWaves;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys);
  // the row this lane loads with instruction j of the wave's k-th tile and
  // its page slot (-1: not scored, -2: bad page)
  auto row_page = [&](int k, int j, size_t* off) {
    const int t = wave + kIdxWaves * k;           // tile in the workgroup
    const int u = 16 * t + j * T::RPI + lane / T::LPR;   // unit of the row (in the wg)
    int pslot, page;
    if constexpr (MODE == kIdxTokens) {
      pslot = (u0 + u) / P - bi0;
      page = k < ntw ? sh.pg[pslot] : -1;
      const int slot = (u0 + u) % P;
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
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      size_t off;
      const int page = row_page(k, j, &off);
      badm |= (uint32_t)(page == -2) << j;
      d[j] = ldg16(kbase + off + 16 * (lane % T::LPR));
    }
    sig = 1.0f;
    if constexpr (MODE == kIdxTokens) {
      if (a.scales) {
        const int t = wave + kIdxWaves * k;
        const int u = u0 + 16 * t + col;
        const int page = k < ntw ? sh.pg[u / P - bi0] : -1;
        sig = a.scales[(size_t)(uint32_t)(page >= 0 ? page : 0) * P + u % P];
      }
    }
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
        uint32_t* tile = sh.tiles[wave][s & 1];
        // stage row-major (rows with a bad page become zeros)
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int row = j * T::RPI + lane / T::LPR;
          *reinterpret_cast<uint4*>(tile + row * T::RW + 4 * (lane % T::LPR)) =
              ((bm >> j) & 1u) ? make_uint4(0, 0, 0, 0) : c[j];
        }
        wave_lds_sync();
        // B operand (key^T): unit `col`, dims 32kq + 8s .. +8 of k-step s
        uint4 kb[4];
        if constexpr (MODE == kIdxTokens) {
          const uint4 x0 = *reinterpret_cast<const uint4*>(tile + col * T::RW + 8 * kq);
          const uint4 x1 = *reinterpret_cast<const uint4*>(tile + col * T::RW + 8 * kq + 4);
          const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            kb[s2] = make_uint4(fp8x2_to_bf16x2(xs[2 * s2], false),
                                fp8x2_to_bf16x2(xs[2 * s2], true),
                                fp8x2_to_bf16x2(xs[2 * s2 + 1], false),
                                fp8x2_to_bf16x2(xs[2 * s2 + 1], true));
        } else {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            kb[s2] = *reinterpret_cast<const uint4*>(tile + col * T::RW + 16 * kq + 4 * s2);
        }
        f32x4_t acc[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          acc[ht] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) acc[ht] = mfma_16x16x32(qa[ht][s2], kb[s2], acc[ht]);
        }
        // s = sum_h w_h max(0, sigma * d_h); lane holds heads 16ht + 4kq + i
        float v = 0.0f;
        if (__ballot(!(sg > 0.0f)) == 0) {   // all scales positive: sigma factors out
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) v = fmaf(wv[ht][i], fmaxf(acc[ht][i], 0.0f), v);
          v = xor_pair_sum<16>(v);
          v = xor_pair_sum<32>(v);
          v *= sg;
        } else {
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) v = fmaf(wv[ht][i], fmaxf(acc[ht][i] * sg, 0.0f), v);
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
          sh.sc[ul] = valid ? v : 0.0f;
        }
      }
    }
  }
  __syncthreads();
  float* srow = a.scores + (size_t)r * a.max_units + u0;
  const int nw = n_units - u0 < upw ? n_units - u0 : upw;
  for (int i = tid; i < nw; i += kIdxThreads) srow[i] = sh.sc[i];
  if constexpr (MODE == kIdxTokens) {
    uint32_t* gh = a.hist + (size_t)r * kIdxBins;
    for (int i = tid; i < kIdxBins; i += kIdxThreads) {
      const uint32_t c = sh.hist[i];
      if (c) atomicAdd(gh + i, c);
    }
  }
}

// ------------------------------------------------------------ token top-k ----

__global__ __launch_bounds__(kIdxThreads) void idx_zero_kernel(uint32_t* hist, uint32_t* ctl,
                                                               int batch) {
  const int n = batch * kIdxBins;
  for (int i = blockIdx.x * kIdxThreads + threadIdx.x; i < n; i += gridDim.x * kIdxThreads)
    hist[i] = 0u;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < batch * 4; i += kIdxThreads) ctl[i] = 0u;
}

struct IdxFinLds {
  uint32_t bm[kIdxMaxWords];
  uint32_t tie[kIdxMaxWords];
  uint32_t ckey[kIdxCandCap];
  int32_t cunit[kIdxCandCap];
  int32_t h2[1024];
};

struct IdxMarkLds {
  union {
    uint32_t hist[kIdxBins];
    IdxFinLds fin;
  } u;
  int red[kIdxWaves];
  int bstar, cabove, cat, kr, nvalid, last, b2, need;
};

// Exclusive prefix sum over the workgroup in thread order; *total = sum.
__device__ __forceinline__ int idx_block_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kIdxWaves; ++w) {
    const int x = red[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// Digit search from the top: the bin b of h[0 .. nbins) (each thread owns
// nbins / kIdxThreads consecutive bins) at which the count of elements in
// bins > b is < need and the count in bins >= b is >= need. Returns (via
// LDS) b and the count above it. need >= 1 and sum(h) >= need.
__device__ __forceinline__ void idx_find_digit(const int32_t* h, int nbins, int need, int* red,
                                               int* b_out, int* above_out) {
  const int per = nbins / kIdxThreads, t = threadIdx.x;
  int mine = 0;
  for (int i = 0; i < per; ++i) mine += h[t * per + i];
  int tot;
  const int excl = idx_block_scan(mine, red, &tot);
  int above = tot - excl - mine;   // elements in bins of higher threads
  if (above < need && above + mine >= need) {
    for (int b = t * per + per - 1; b >= t * per; --b) {
      if (above + h[b] >= need) {
        *b_out = b;
        *above_out = above;
        break;
      }
      above += h[b];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int idx_token_of(const IndexerArgs& a, const IdxUnits& g, int r,
                                           int u) {
  if (g.ncand < 0) return u;
  const int P = a.b.page_size;
  return a.cand_blocks[(size_t)r * a.cand_cap + u / P] * P + u % P;
}

__global__ __launch_bounds__(kIdxThreads) void idx_mark_kernel(IndexerArgs a) {
  __shared__ IdxMarkLds sh;
  const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const IdxUnits g = idx_units(a, r);
  const int nwords_row = a.max_units / 32;
  uint32_t* bmrow = a.bitmap + (size_t)r * nwords_row;
  uint32_t* ctl = a.ctl + (size_t)r * 4;
  const float* srow = a.scores + (size_t)r * a.max_units;

  // 1. threshold bin from the request's histogram
  const uint32_t* gh = a.hist + (size_t)r * kIdxBins;
  for (int i = tid; i < kIdxBins; i += kIdxThreads) sh.u.hist[i] = gh[i];
  if (tid == 0) {
    sh.bstar = kIdxBins;   // nothing definite, no candidates
    sh.cabove = 0;
    sh.cat = 0;
  }
  __syncthreads();
  {
    int mine = 0;
    constexpr int per = kIdxBins / kIdxThreads;
    for (int i = 0; i < per; ++i) mine += (int)sh.u.hist[tid * per + i];
    int tot;
    const int excl = idx_block_scan(mine, sh.red, &tot);
    const int kr = a.topk < tot ? a.topk : tot;
    if (tid == 0) {
      sh.kr = kr;
      sh.nvalid = tot;
      if (kr >= tot && tot > 0) sh.bstar = -1;   // every valid unit is selected
    }
    if (kr > 0 && kr < tot) {
      int above = tot - excl - mine;
      if (above < kr && above + mine >= kr) {
        for (int b = tid * per + per - 1; b >= tid * per; --b) {
          const int hb = (int)sh.u.hist[b];
          if (above + hb >= kr) {
            sh.bstar = b;
            sh.cabove = above;
            sh.cat = hb;
            break;
          }
          above += hb;
        }
      }
    }
  }
  __syncthreads();
  const int bstar = sh.bstar, cat = sh.cat;
  const bool collect = bstar >= 0 && bstar < kIdxBins && cat <= kIdxCandCap;

  // 2. mark this chunk's units: selected bits, and candidates in bin b*
  const int cu0 = chunk * kIdxMarkUnits;
  for (int it = 0; it < kIdxMarkUnits / kIdxThreads; ++it) {
    const int ub = cu0 + it * kIdxThreads + wave * kWave;   // wave's 64 units
    if (ub >= g.n) break;                                    // uniform per wave
    const int u = ub + lane;
    int tok;
    const bool valid = idx_unit_block(a, g, r, u, &tok) >= 0;
    uint32_t key = 0u, bin = 0u;
    if (valid) {
      key = score_key(srow[u]);
      bin = idx_bin(key);
    }
    const bool def = valid && (bstar < 0 || (int)bin > bstar);
    const bool cnd = collect && valid && (int)bin == bstar;
    const unsigned long long dm = __ballot(def);
    if (lane == 0) {
      st_dev(bmrow + ub / 32, (uint32_t)dm);
      st_dev(bmrow + ub / 32 + 1, (uint32_t)(dm >> 32));
    }
    const unsigned long long cm = __ballot(cnd);
    if (cm) {
      int base = 0;
      if (lane == 0) base = (int)atomicAdd(ctl, (uint32_t)__popcll(cm));
      base = __shfl(base, 0);
      if (cnd) {
        const int pos = base + mbcnt(cm);
        if (pos < kIdxCandCap) st_dev(a.cand + (size_t)r * kIdxCandCap + pos, make_uint2(key, (uint32_t)u));
      }
    }
  }
  // 3. arrival; the last workgroup of the request finishes it (every thread's
  // bitmap and candidate stores are complete and visible device-wide before
  // the workgroup's arrival is counted)
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ctl + 1, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh.last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!sh.last) return;
  __threadfence();

  IdxFinLds& f = sh.u.fin;   // the histogram is no longer needed
  const int kr = sh.kr;
  const int nwr = (g.n + 31) / 32;
  for (int w = tid; w < nwr; w += kIdxThreads) {
    f.bm[w] = ld_dev(bmrow + w);
    f.tie[w] = 0u;
  }
  int ties_to_take = 0;
  if (bstar >= 0 && bstar < kIdxBins) {
    const int need = kr - sh.cabove;   // >= 1 units of bin b* to select
    int nc = collect ? (int)ld_dev(ctl) : 0;
    nc = nc < kIdxCandCap ? nc : kIdxCandCap;
    if (collect) {
      for (int i = tid; i < nc; i += kIdxThreads) {
        const uint2 c = ld_dev(a.cand + (size_t)r * kIdxCandCap + i);
        f.ckey[i] = c.x;
        f.cunit[i] = (int)c.y;
      }
    }
    // visit every candidate (unit in bin b*): from LDS, or by streaming the
    // request's scores when they did not fit
    auto for_each = [&](auto&& fn) {
      if (collect) {
        for (int i = tid; i < nc; i += kIdxThreads) fn(f.ckey[i], f.cunit[i]);
      } else {
        for (int u = tid; u < g.n; u += kIdxThreads) {
          int tok;
          if (idx_unit_block(a, g, r, u, &tok) < 0) continue;
          const uint32_t key = score_key(srow[u]);
          if ((int)idx_bin(key) == bstar) fn(key, u);
        }
      }
    };
    // second digit: key bits [19:10]
    for (int i = tid; i < 1024; i += kIdxThreads) f.h2[i] = 0;
    __syncthreads();
    for_each([&](uint32_t key, int) { atomicAdd(&f.h2[(key >> 10) & 1023u], 1); });
    __syncthreads();
    idx_find_digit(f.h2, 1024, need, sh.red, &sh.b2, &sh.need);
    const int b2 = sh.b2, need2 = need - sh.need;
    // third digit: key bits [9:0] of the candidates with digit 2 == b2
    for (int i = tid; i < 1024; i += kIdxThreads) f.h2[i] = 0;
    __syncthreads();
    for_each([&](uint32_t key, int) {
      if ((int)((key >> 10) & 1023u) == b2) atomicAdd(&f.h2[key & 1023u], 1);
    });
    __syncthreads();
    idx_find_digit(f.h2, 1024, need2, sh.red, &sh.b2, &sh.need);
    const uint32_t theta = ((uint32_t)bstar << 20) | ((uint32_t)b2 << 10) | (uint32_t)sh.b2;
    ties_to_take = need2 - sh.need;
    for_each([&](uint32_t key, int u) {
      if (key > theta) atomicOr(&f.bm[u >> 5], 1u << (u & 31));
      else if (key == theta) atomicOr(&f.tie[u >> 5], 1u << (u & 31));
    });
    __syncthreads();
  } else {
    __syncthreads();
  }

  // 4. emit in ascending unit order: the bitmap plus the first ties
  const int wpt = (nwr + kIdxThreads - 1) / kIdxThreads;
  const int w0 = tid * wpt, w1 = w0 + wpt < nwr ? w0 + wpt : nwr;
  int tcount = 0;
  for (int w = w0; w < w1; ++w) tcount += __popc(f.tie[w]);
  int ttot;
  int tpre = idx_block_scan(tcount, sh.red, &ttot);
  int scount = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t x = f.tie[w], kept = 0u;
    int take = ties_to_take - tpre;
    const int pc = __popc(x);
    take = take < 0 ? 0 : (take > pc ? pc : take);
    for (int i = 0; i < take; ++i) {
      const uint32_t low = x & (0u - x);
      kept |= low;
      x ^= low;
    }
    tpre += pc;
    const uint32_t sel = f.bm[w] | kept;
    f.bm[w] = sel;
    scount += __popc(sel);
  }
  int stot;
  int pos = idx_block_scan(scount, sh.red, &stot);
  int32_t* out = a.selected + (size_t)r * a.max_selected;
  for (int w = w0; w < w1; ++w) {
    uint32_t x = f.bm[w];
    while (x) {
      const int b = __ffs(x) - 1;
      x &= x - 1u;
      if (pos < a.max_selected) out[pos] = idx_token_of(a, g, r, 32 * w + b);
      ++pos;
    }
  }
  for (int i = stot + tid; i < a.max_selected; i += kIdxThreads) out[i] = -1;
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

hipError_t launch_indexer_token_select(const IndexerArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(idx_zero_kernel, dim3(16), dim3(kIdxThreads), 0, st, a.hist, a.ctl,
                     a.b.batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_score_mode<kIdxTokens>(a, st);
  if (e != hipSuccess) return e;
  dim3 grid((a.max_units + kIdxMarkUnits - 1) / kIdxMarkUnits, a.b.batch);
  hipLaunchKernelGGL(idx_mark_kernel, grid, dim3(kIdxThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ls

// Standalone GQA block-scoring kernel (see dev_score.h for the method and the
// memory walk): one wave per kBlocksPerWave consecutive blocks of a request.
#include "dev_score.h"

namespace ls {

template <int D, int HKV, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  using S = ScoreShape<D, HKV, G>;
  __shared__ ScoreLds<D, HKV, G> st[4];
  const int r = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
  const int wb0 = (blockIdx.x * 4 + wave) * S::kBlocksPerWave;
  score_wave<D, HKV, G, false>(a, r, geo, wb0, lane, st[wave]);
}

template <int D, int HKV, int G>
static hipError_t launch(const ScoreArgs& a, hipStream_t st) {
  constexpr int kPerWG = 4 * ScoreShape<D, HKV, G>::kBlocksPerWave;
  dim3 grid((a.b.max_blocks + kPerWG - 1) / kPerWG, a.b.batch);
  hipLaunchKernelGGL((score_kernel<D, HKV, G>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_g(const ScoreArgs& a, hipStream_t st) {
  switch (a.num_kv_heads) {
    case 1: return launch<D, 1, G>(a, st);
    case 2: return launch<D, 2, G>(a, st);
    case 4: return launch<D, 4, G>(a, st);
    case 8: return launch<D, 8, G>(a, st);
    case 16: return launch<D, 16, G>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_d(const ScoreArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<D, 1>(a, st);
    case 2: return launch_g<D, 2>(a, st);
    case 4: return launch_g<D, 4>(a, st);
    case 8: return launch_g<D, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

// GQA groups of 1, 2, 4 or 8 query heads per kv head.
hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  return a.head_dim == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}

}  // namespace ls

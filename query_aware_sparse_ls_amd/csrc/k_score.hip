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

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  const int D = a.head_dim, H = a.num_kv_heads;
  if (D == 128) {
    switch (H) {
      case 1: return launch<128, 1, 4>(a, st);
      case 2: return launch<128, 2, 4>(a, st);
      case 4: return launch<128, 4, 4>(a, st);
      case 8: return launch<128, 8, 4>(a, st);
      case 16: return launch<128, 16, 4>(a, st);
    }
  } else {
    switch (H) {
      case 1: return launch<64, 1, 4>(a, st);
      case 2: return launch<64, 2, 4>(a, st);
      case 4: return launch<64, 4, 4>(a, st);
      case 8: return launch<64, 8, 4>(a, st);
      case 16: return launch<64, 16, 4>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ls

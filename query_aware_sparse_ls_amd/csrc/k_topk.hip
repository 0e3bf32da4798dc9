// Standalone top-k kernel: one workgroup per (request, kv head)
// (see dev_topk.h for the method).
#include "dev_topk.h"

namespace ls {

// The candidates' scores are first copied into LDS with coalesced loads
// (consecutive lanes, consecutive scores; one pad word after every 16): the
// top-k's thread-owns-PER-consecutive-candidates layout read straight from
// memory would have each lane touch its own line.
template <int PER, int NT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  __shared__ TopkLds sh;
  __shared__ float stage[PER * NT + PER * NT / 16];
  const int g = blockIdx.x, r = blockIdx.y;
  const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
  const int item = r * a.num_kv_heads + g;
  const float* srow = a.scores + (size_t)item * a.b.max_blocks + geo.c0;
  const int n = geo.c1 - geo.c0;
  float v[PER];   // every load issued before any is stored
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int i = threadIdx.x + m * NT;
    v[m] = i < n ? srow[i] : 0.0f;
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int i = threadIdx.x + m * NT;
    stage[i + (i >> 4)] = v[m];
  }
  __syncthreads();
  topk_wg<PER, NT, true>(stage, geo, topk_budget(a, geo),
                         a.selected + (size_t)item * a.max_selected, a.max_selected,
                         a.selected_count + item, sh);
}

template <int PER, int NT>
static hipError_t launch(const TopkArgs& a, hipStream_t st) {
  dim3 grid(a.num_kv_heads, a.b.batch);
  hipLaunchKernelGGL((topk_kernel<PER, NT>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

// 256 threads per workgroup while there are many (request, kv head) pairs or
// few blocks; 1024 (16 candidates per thread) for long requests in small
// batches, where a few workgroups hold the whole selection.
hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int pairs = a.num_kv_heads * a.b.batch;
  if (a.b.max_blocks > 2048 && pairs < 128) {
    const int per = (a.b.max_blocks + 1023) / 1024;
    if (per <= 4) return launch<4, 1024>(a, st);
    if (per <= 8) return launch<8, 1024>(a, st);
    return launch<16, 1024>(a, st);
  }
  const int per = (a.b.max_blocks + kTopkThreads - 1) / kTopkThreads;
  if (per <= 2) return launch<2, kTopkThreads>(a, st);
  if (per <= 4) return launch<4, kTopkThreads>(a, st);
  if (per <= 8) return launch<8, kTopkThreads>(a, st);
  if (per <= 16) return launch<16, kTopkThreads>(a, st);
  if (per <= 32) return launch<32, kTopkThreads>(a, st);
  return launch<64, kTopkThreads>(a, st);
}

}  // namespace ls

// Standalone top-k kernel: one 256-thread workgroup per (request, kv head)
// (see dev_topk.h for the method).
#include "dev_topk.h"

namespace ls {

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkLds sh;
  const int g = blockIdx.x, r = blockIdx.y;
  const ReqGeom geo = req_geom(a.b, r, a.n_sink, a.n_recent);
  const int item = r * a.num_kv_heads + g;
  const float* srow = a.scores + (size_t)item * a.b.max_blocks + geo.c0;
  topk_wg<PER>(srow, geo, topk_budget(a, geo), a.selected + (size_t)item * a.max_selected,
               a.max_selected, a.selected_count + item, sh);
}

template <int PER>
static hipError_t launch(const TopkArgs& a, hipStream_t st) {
  dim3 grid(a.num_kv_heads, a.b.batch);
  hipLaunchKernelGGL((topk_kernel<PER>), grid, dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int per = (a.b.max_blocks + kTopkThreads - 1) / kTopkThreads;
  if (per <= 2) return launch<2>(a, st);
  if (per <= 4) return launch<4>(a, st);
  if (per <= 8) return launch<8>(a, st);
  if (per <= 16) return launch<16>(a, st);
  if (per <= 32) return launch<32>(a, st);
  return launch<64>(a, st);
}

}  // namespace ls

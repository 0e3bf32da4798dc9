// Standalone split-K attention and combine kernels (see dev_attn.h for the
// method, the memory walk and the merge).
#include "dev_attn.h"

namespace ls {

template <int D, int G>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  __shared__ AttnLds<D, G> sh;
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const ReqGeom geo = req_geom(a.b, r, 0, 0);
  attn_split<D, G, kAttnBlocksPerSplit, false>(a, geo, r, g, s, sh);
}

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.b.batch * a.num_q_heads) return;
  combine_head<D, false>(a, item, threadIdx.x & 63);
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.num_splits, a.num_kv_heads, a.b.batch);
  switch (a.num_q_heads / a.num_kv_heads) {   // GQA groups of 1, 2, 4 or 8
    case 1: hipLaunchKernelGGL((attn_split_kernel<D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_split_kernel<D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_split_kernel<D, 4>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_split_kernel<D, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items = a.b.batch * a.num_q_heads;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((items + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st) {
  const int items = a.b.batch * a.num_q_heads;
  if (a.head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), dim3((items + 3) / 4), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), dim3((items + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.head_dim == 128) return launch_d<128>(a, st);
  return launch_d<64>(a, st);
}

}  // namespace ls

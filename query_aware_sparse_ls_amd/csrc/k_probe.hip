// Measurement reference: a plain streaming read of a device buffer, the
// bandwidth a kernel of this library is compared with on the same GPU
// (ByteCross §4.4 and App. D price a decode step against the bandwidth the
// memory actually delivers). Every 16-byte word is read once, non-temporal,
// four loads in flight per thread. The 32-bit words are XOR-folded so that
// no load is dead: each workgroup writes the XOR of the words it read, so
// the XOR of all sink words is the XOR of the whole buffer.
#include "ls_internal.h"

namespace ls {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 4;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                                    size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = blockIdx.x * (size_t)kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) v[u] = ldg16_stream(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ldg16_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  __shared__ uint32_t part[kProbeThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / kWave; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t st) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st,
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace ls

// Measurement reference: a plain streaming read of a device buffer, the
// bandwidth a kernel of this library is compared with on the same GPU
// (ByteCross §4.4 and App. D price a decode step against the bandwidth the
// memory actually delivers). Every 16-byte word is read once, non-temporal.
// The buffer is cut into 4 KB chunks dealt to the waves round-robin; a wave
// reads a whole chunk per round (its 64 lanes x 16 bytes x 4 loads in
// flight). On MI355X this form read 6.5-6.7 TB/s over 138 MB-2 GB buffers,
// where a grid-stride loop of 16-byte loads (each wave instruction 1 KB,
// consecutive ones a grid apart) read 5.6-6.0 TB/s. The 32-bit words are
// XOR-folded so that no load is dead: each workgroup writes the XOR of the
// words it read, so the XOR of all sink words is the XOR of the whole buffer.
#include "ls_internal.h"

namespace ls {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 4;                        // 16-byte loads per lane and round
constexpr int kProbeChunk16 = kWave * kProbeInFlight;    // 16-byte words per chunk (4 KB)

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                                    size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  constexpr int NW = kProbeThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const size_t nwaves = (size_t)gridDim.x * NW;
  const size_t nchunks = (n16 + kProbeChunk16 - 1) / kProbeChunk16;
  uint32_t acc = 0;
  for (size_t c = (size_t)blockIdx.x * NW + threadIdx.x / kWave; c < nchunks; c += nwaves) {
    const size_t w0 = c * kProbeChunk16 + lane;
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const size_t w = w0 + (size_t)u * kWave;
      v[u] = w < n16 ? ldg16_stream(p + w) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
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

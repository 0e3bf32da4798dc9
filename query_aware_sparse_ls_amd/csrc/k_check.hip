// Debug check of a ragged batch's device data: the CSR page table and the
// lengths that every kernel of the library reads (the Vortex post's vTensor:
// an index-pointer array over a page list, "Why New Ideas Are Hard to
// Deploy"). The kernels already clamp what breaks the contract (ReqGeom);
// this check reports it. One workgroup walks the requests in order; per
// request it tests the index pointers, the length against the page list and
// max_blocks, and every page id of the blocks a kernel would read (those
// below min(blocks of the length, the list's length, max_blocks)) against
// [0, num_pages). It reads only entries inside each request's stated list.
#include <climits>

#include "ls_internal.h"

namespace ls {

namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void batch_check_kernel(BatchArgs b, int32_t* report,
                                                                    int accumulate) {
  __shared__ int s_kinds, s_bad, s_first;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_kinds = 0;
    s_bad = 0;
    s_first = INT_MAX;
  }
  __syncthreads();
  for (int r = 0; r < b.batch; ++r) {
    const int p0 = b.indptr[r], p1 = b.indptr[r + 1];
    const int L = b.seq_lens[r];
    int kinds = 0;
    if (p0 < 0 || p1 < p0) kinds |= LS_BATCH_BAD_INDPTR;
    if (L < 0) kinds |= LS_BATCH_NEGATIVE_LENGTH;
    const long long list = (kinds & LS_BATCH_BAD_INDPTR) ? 0 : (long long)p1 - p0;
    const long long nb = L > 0 ? ((long long)L + b.page_size - 1) / b.page_size : 0;
    if (nb > list) kinds |= LS_BATCH_LENGTH_BEYOND_PAGES;
    if (nb > b.max_blocks) kinds |= LS_BATCH_LENGTH_BEYOND_MAX_BLOCKS;
    long long used = nb < list ? nb : list;
    used = used < b.max_blocks ? used : b.max_blocks;
    int bad = 0;
    for (long long j = tid; j < used; j += kCheckThreads) {
      const int pg = b.indices[p0 + j];
      bad |= (pg < 0 || pg >= b.num_pages) ? 1 : 0;
    }
    if (__syncthreads_or(bad)) kinds |= LS_BATCH_PAGE_OUT_OF_RANGE;
    if (tid == 0 && kinds) {
      s_kinds |= kinds;
      s_bad += 1;
      s_first = r < s_first ? r : s_first;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (accumulate) {
      // library debug words: kinds seen, calls with a violation, violating
      // requests, calls checked
      atomicOr(report + 0, s_kinds);
      atomicAdd(report + 1, s_bad ? 1 : 0);
      atomicAdd(report + 2, s_bad);
      atomicAdd(report + 3, 1);
    } else {
      report[0] = s_kinds;
      report[1] = s_bad;
      report[2] = s_bad ? s_first : -1;
      report[3] = b.batch;
    }
  }
}

}  // namespace

hipError_t launch_batch_check(const BatchArgs& b, int32_t* report, bool accumulate,
                              hipStream_t stream) {
  batch_check_kernel<<<1, kCheckThreads, 0, stream>>>(b, report, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace ls

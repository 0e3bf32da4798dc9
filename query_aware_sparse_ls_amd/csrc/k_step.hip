// Fused decode step: block scoring, top-k selection and split-K attention of
// a whole batch in ONE persistent kernel launch.
//
// Same method as the separate calls (dev_score.h, dev_topk.h, dev_attn.h);
// what the fusion adds is overlap. The Vortex post plans each decode step's
// work across requests and fuses operators so block scores never make a round
// trip through GPU memory ("Making it fast"); on this chip the larger win is
// that one request's selection and attention can run while other requests
// are still being scored, so the dependent chain (scores -> top-k ->
// selection -> page ids -> K/V) never leaves HBM idle, and no kernel
// boundary or launch tail is paid between the steps.
//
// Scheduling: requests are dealt to NQ work queues (request r -> queue
// r % NQ). A queue's tasks, in ticket order, are: the score tasks of its
// requests, then their top-k tasks, then their attention split tasks.
// Persistent workgroups take tickets from their home queue (blockIdx.x % NQ)
// and move on to the other queues when it runs dry.
//  * score task (r, chunk): scores the chunk's candidate blocks and counts
//    itself done for request r.
//  * top-k task (r, g): waits until every score task of r is done, selects,
//    and publishes a ready flag for (r, g).
//  * attention task (r, g, split): waits for the (r, g) ready flag, then runs
//    the split; the LAST split of (r, g) to finish merges the splits.
// A task only ever waits for tasks with a smaller ticket in the same queue,
// which were taken earlier by running workgroups that never wait on later
// tickets, so the oldest unfinished task can always progress: no deadlock,
// whether or not every workgroup is resident. Waits are bounded; a wait that
// runs out sets an error word instead of hanging.
//
// Cross-workgroup hand-offs: the handed-over data (scores, selections, split
// partials) is stored and loaded with device-coherent accesses (st_dev /
// ld_dev); a producer waits for its stores to complete before the arrival
// atomic that publishes them, so no whole-cache write-back or invalidate is
// needed. The control block (tickets and counters) must be zero before the
// first launch; the last workgroup to exit zeroes it again.
#include "dev_attn.h"
#include "dev_score.h"
#include "dev_topk.h"

namespace ls {

constexpr int kNQ = 8;                 // work queues
constexpr int kSpinLimit = 1 << 22;    // polls before giving up (~0.1 s)

struct StepCtl {
  unsigned int ticket[kNQ][32];        // one 128-byte line per queue
  unsigned int exited;
  unsigned int error;
  unsigned int pad[30];
  // followed by: score_done[B], ready[B * Hkv], attn_done[B * Hkv]
};

struct StepArgs {
  ScoreArgs sc;
  TopkArgs tk;
  AttnArgs at;
  StepCtl* ctl;
  unsigned int* score_done;
  unsigned int* ready;
  unsigned int* attn_done;
  int score_tasks_per_req;   // chunks of kStepScoreBlocks
};

__device__ __forceinline__ unsigned int load_agent(const unsigned int* p) {
  return ld_dev(p);
}

template <int D, int HKV, int G, int MAXC>
union StepLds {
  AttnLds<D, G> attn;
  TopkLds topk;
  ScoreLds<D, HKV, G> score[4];
};

template <int D, int HKV, int G, int MAXC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_step_kernel(StepArgs a) {
  using SS = ScoreShape<D, HKV, G>;
  constexpr int kChunk = 4 * SS::kBlocksPerWave;   // blocks per score task
  __shared__ StepLds<D, HKV, G, MAXC> sh;
  __shared__ int s_task;
  __shared__ int s_flag;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.sc.b.batch;
  const int S = a.at.num_splits;
  const int home = blockIdx.x % kNQ;

  for (int qi = 0; qi < kNQ;) {
    const int q = (home + qi) % kNQ;
    const int nreq = q < B ? (B - 1 - q) / kNQ + 1 : 0;
    const int n_score = nreq * a.score_tasks_per_req;
    const int n_topk = nreq * HKV;
    const int n_total = n_score + n_topk + nreq * HKV * S;
    if (tid == 0) s_task = (int)atomicAdd(&a.ctl->ticket[q][0], 1u);
    __syncthreads();
    const int t = s_task;
    __syncthreads();
    if (t >= n_total) {
      ++qi;
      continue;
    }
    if (t < n_score) {
      // ---------------------------------------------------- score task
      const int r = q + (t / a.score_tasks_per_req) * kNQ;
      const int chunk = t % a.score_tasks_per_req;
      const ReqGeom geo = req_geom(a.sc.b, r, a.sc.n_sink, a.sc.n_recent);
      score_wave<D, HKV, G, true>(a.sc, r, geo, chunk * kChunk + wave * SS::kBlocksPerWave, lane,
                                  sh.score[wave]);
      wait_stores();
      __syncthreads();
      if (tid == 0) atomicAdd(&a.score_done[r], 1u);
    } else if (t < n_score + n_topk) {
      // ----------------------------------------------------- top-k task
      const int u = t - n_score;
      const int r = q + (u / HKV) * kNQ;
      const int g = u % HKV;
      const int item = r * HKV + g;
      if (tid == 0) {
        int spins = 0;
        while (load_agent(&a.score_done[r]) < (unsigned int)a.score_tasks_per_req) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpinLimit) {
            atomicOr(&a.ctl->error, 1u);
            break;
          }
        }
      }
      __syncthreads();
      const ReqGeom geo = req_geom(a.tk.b, r, a.tk.n_sink, a.tk.n_recent);
      const float* srow = a.tk.scores + (size_t)item * a.tk.b.max_blocks + geo.c0;
      topk_wg<MAXC / kTopkThreads, true>(srow, geo, topk_budget(a.tk, geo),
                                   a.tk.selected + (size_t)item * a.tk.max_selected,
                                   a.tk.max_selected, a.tk.selected_count + item, sh.topk);
      wait_stores();
      __syncthreads();
      if (tid == 0) st_dev(&a.ready[item], 1u);
    } else {
      // ------------------------------------------------ attention task
      const int u = t - n_score - n_topk;
      const int r = q + (u / (HKV * S)) * kNQ;
      const int g = (u / S) % HKV;
      const int s = u % S;
      const int item = r * HKV + g;
      if (tid == 0) {
        int spins = 0;
        while (load_agent(&a.ready[item]) == 0u) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kSpinLimit) {
            atomicOr(&a.ctl->error, 1u);
            break;
          }
        }
      }
      __syncthreads();
      const ReqGeom geo = req_geom(a.at.b, r, 0, 0);
      const SelRow sr = sel_row<true>(a.at, geo, r, g);
      const int lo = (int)(((long long)s * sr.cnt) / S);
      const int hi = (int)(((long long)(s + 1) * sr.cnt) / S);
      attn_split<D, G, kAttnBlocksPerSplit, true>(a.at, geo, sr, r, g, s, lo, hi, sh.attn);
      wait_stores();        // every wave's partial stores, before the arrival below
      __syncthreads();
      if (tid == 0) {
        const unsigned int old = atomicAdd(&a.attn_done[item], 1u);
        s_flag = old == (unsigned int)(S - 1);
      }
      __syncthreads();
      if (s_flag) {
        combine_head<D, true>(a.at, r * a.at.num_q_heads + g * G + wave, lane);   // G = 4 waves
        __syncthreads();
      }
    }
  }

  // the last workgroup out zeroes the control block for the next launch
  __syncthreads();
  if (tid == 0) {
    const unsigned int old = atomicAdd(&a.ctl->exited, 1u);
    s_flag = old == gridDim.x - 1;
  }
  __syncthreads();
  if (s_flag) {
    for (int i = tid; i < kNQ; i += 256) st_dev(&a.ctl->ticket[i][0], 0u);
    for (int i = tid; i < B; i += 256) st_dev(&a.score_done[i], 0u);
    for (int i = tid; i < B * HKV; i += 256) { st_dev(&a.ready[i], 0u); st_dev(&a.attn_done[i], 0u); }
    if (tid == 0) st_dev(&a.ctl->exited, 0u);
  }
}

size_t step_ctl_bytes(int batch, int hkv) {
  return (sizeof(StepCtl) + sizeof(unsigned int) * ((size_t)batch + 2 * (size_t)batch * hkv) +
          255) / 256 * 256;
}

template <int D, int HKV, int MAXC>
static hipError_t launch_step_t(const StepLaunch& L, hipStream_t st) {
  constexpr int G = 4;
  auto kern = decode_step_kernel<D, HKV, G, MAXC>;
  static int per_cu = 0, cus = 0;
  if (per_cu == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
  }
  using SS = ScoreShape<D, HKV, G>;
  StepArgs a;
  a.sc = L.sc;
  a.tk = L.tk;
  a.at = L.at;
  a.ctl = static_cast<StepCtl*>(L.ctl);
  unsigned int* words = reinterpret_cast<unsigned int*>(a.ctl + 1);
  const int B = L.sc.b.batch;
  a.score_done = words;
  a.ready = words + B;
  a.attn_done = words + B + B * HKV;
  a.score_tasks_per_req = (L.sc.b.max_blocks + 4 * SS::kBlocksPerWave - 1) / (4 * SS::kBlocksPerWave);
  const long long tasks = (long long)B * (a.score_tasks_per_req + HKV + HKV * L.at.num_splits);
  long long grid = (long long)per_cu * cus;
  if (grid > tasks) grid = tasks;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

bool step_supported(int head_dim, int hkv, int max_blocks) {
  return (head_dim == 128 || head_dim == 64) && (hkv == 2 || hkv == 4 || hkv == 8) &&
         max_blocks <= 4096;
}

hipError_t launch_step(const StepLaunch& L, hipStream_t st) {
  const int D = L.sc.head_dim, H = L.sc.num_kv_heads, n = L.sc.b.max_blocks;
#define LS_STEP_CASE(DD, HH)                                              \
  if (D == DD && H == HH) {                                               \
    if (n <= 512) return launch_step_t<DD, HH, 512>(L, st);               \
    if (n <= 2048) return launch_step_t<DD, HH, 2048>(L, st);             \
    return launch_step_t<DD, HH, 4096>(L, st);                            \
  }
  LS_STEP_CASE(128, 8)
  LS_STEP_CASE(128, 4)
  LS_STEP_CASE(128, 2)
  LS_STEP_CASE(64, 8)
  LS_STEP_CASE(64, 4)
  LS_STEP_CASE(64, 2)
#undef LS_STEP_CASE
  return hipErrorInvalidValue;
}

}  // namespace ls

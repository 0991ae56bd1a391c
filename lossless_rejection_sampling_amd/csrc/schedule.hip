// Hardware-aware prefix scheduler ("DSpark, la bozza che sa quando fermarsi",
// section "Verificare meglio, non di più": a_j = prod_{i<=j} c_i, Theta =
// tau * SPS(B), candidates admitted in decreasing a while Theta grows, with an
// early stop at the first candidate that does not raise it), and its variants:
// Sequential Temperature Scaling of the scores (same section), the production
// rule that takes the best cut without the early stop (section "Che cosa resta
// da verificare"), and the fixed-length and fixed-threshold baselines.
//
// The admitted prefix is found without sorting.  The position (rank) m of a
// candidate in the order (Q desc, request asc, position asc) is the number of
// keys ordered before it, and tau_m - B 2^32 is the sum of their Q; both come
// from one pass over all keys, in exact integer arithmetic, so the test of every
// candidate is evaluated independently:
//   1. every workgroup forms all keys in LDS (a lane per request: optional
//      temperature scaling, fp32 prefix products left to right, Q = floor(a *
//      2^32)) and the step-time table; the fixed and threshold rules finish here;
//   2. 16 lanes per candidate count and sum the keys before it; the early-stop
//      rule runs its test in fp64 in the stated order and a failing candidate
//      lowers the device-wide first failure (an atomic max of kNoFail - m); the
//      best-cut rule stores Theta after the candidate, theta[m + 1];
//   3. ranks go to the workspace; the last workgroup to finish (a ticket
//      counter) finds the cut (first failure, or the first largest Theta), sets
//      budget[b] = number of b's candidates ranked before it, and resets the
//      counter and the failure word.
#include <map>
#include <mutex>

#include "schedule_body.hpp"

namespace dspark {
namespace {

__global__ __launch_bounds__(kThreads) void schedule_kernel(ScheduleArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  schedule_block(a, blockIdx.x, gridDim.x, smem);
}

}  // namespace

int schedule_groups(const ScheduleArgs& a) {
  const bool ranked = a.rule == DSPARK_SCHED_EARLY_STOP || a.rule == DSPARK_SCHED_ARGMAX;
  return ranked ? (a.B * a.gamma + kCandPerGroup - 1) / kCandPerGroup : 1;
}

size_t schedule_lds_bytes(const ScheduleArgs& a) {
  return (size_t)((a.B * a.gamma + 1) & ~1) * 8 + (size_t)a.n_points * 16;
}

// ---------------------------------------------------------------------------
// Scratch of dspark_schedule_static, for callers that cannot allocate device
// memory: one array per GPU the library runs on, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host that name is
// a stand-in, not a device address): it looks up the array's device address
// once per device with hipGetSymbolAddress and uses that.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScheduleBytes];

__global__ void clear_header_kernel(uint32_t* words, int n) {
  if ((int)threadIdx.x < n) words[threadIdx.x] = 0u;
}

hipError_t static_schedule_scratch(void** ptr, hipStream_t s) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> device address of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  // the header words (status, ticket, first failure, ...) start at zero; every
  // call leaves its counters at zero again.  A kernel, not a memset, so that a
  // first call made under stream capture records no memset node.
  clear_header_kernel<<<1, 64, 0, s>>>(static_cast<uint32_t*>(p), 64);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  addr.emplace(dev, p);
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
  const size_t lds = schedule_lds_bytes(a);
  // dynamic LDS above 64 KB: 80 KB at B gamma = 8192 with a 1024-point table
  int unused = 0;
  const hipError_t e =
      kernel_setup(reinterpret_cast<const void*>(&schedule_kernel), kThreads, 8192 * 8 + 1024 * 16, &unused);
  if (e != hipSuccess) return e;
  launch(&schedule_kernel, schedule_groups(a), kThreads, lds, s, a);
  return hipGetLastError();
}

}  // namespace dspark

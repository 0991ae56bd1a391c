// Hardware-aware prefix scheduler ("DSpark, la bozza che sa quando fermarsi",
// section "Verificare meglio, non di più": a_j = prod_{i<=j} c_i, Theta =
// tau * SPS(B), candidates admitted in decreasing a while Theta grows, with an
// early stop at the first candidate that does not raise it).
//
// One workgroup of 1024 threads:
//   1. a lane per request forms the prefix products in fp32, left to right,
//      and the integer keys Q = floor(a * 2^32);
//   2. the (Q desc, request asc, position asc) keys are sorted in LDS
//      (bitonic network);
//   3. every thread owns a run of consecutive sorted candidates: an integer
//      scan gives tau before each candidate exactly, so the admission test of
//      every candidate is evaluated at once, in fp64 in the stated order;
//   4. the first failing candidate ends the admitted prefix; budgets count the
//      admitted candidates of each request.
#include <math.h>

#include "dspark.h"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxKeys = 8192;
constexpr int kMaxPoints = 1024;

#pragma clang fp contract(off)

// 1/SPS at a verify batch of N tokens (see the ABI header for the rule), from
// the table held in LDS: batch sizes Bs and step times ts = 1/SPS.  The
// segment is the last i <= np-2 with Bs[i] <= N (binary search).
__device__ double step_time(double N, const double* Bs, const double* ts, int np) {
  if (N <= Bs[0]) return ts[0];
  int lo = 0, hi = np - 2;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (Bs[mid] <= N) lo = mid;
    else hi = mid - 1;
  }
  const double frac = (N - Bs[lo]) / (Bs[lo + 1] - Bs[lo]);
  const double dt = ts[lo + 1] - ts[lo];
  const double inc = dt * frac;
  return ts[lo] + inc;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(ScheduleArgs a) {
  __shared__ unsigned long long keys[kMaxKeys];
  __shared__ unsigned long long part[kThreads];
  __shared__ double tB[kMaxPoints], tT[kMaxPoints];
  __shared__ int first_fail;
  const int tid = threadIdx.x, B = a.B, gamma = a.gamma, np = a.n_points;
  const int nk = B * gamma;
  int M = 1;
  while (M < nk) M <<= 1;

  for (int i = tid; i < np; i += kThreads) {
    tB[i] = a.sps_B[i];
    tT[i] = 1.0 / a.sps_val[i];
  }
  bool bad = false;
  for (int b = tid; b < B; b += kThreads) {
    float c[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = j < gamma ? a.conf[(size_t)b * gamma + j] : 0.5f;
    float acc = 1.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= gamma) break;
      float cj = c[j];
      if (!(cj > 0.0f && cj < 1.0f)) {
        bad = true;
        cj = cj > 0.0f ? 0x1.fffffep-1f : 0x1p-126f;  // clamp into (0, 1); NaN -> tiny
      }
      acc = acc * cj;
      const unsigned long long q = (unsigned long long)floor((double)acc * 4294967296.0);
      keys[b * gamma + j] = ((0xFFFFFFFFull - q) << 32) | ((unsigned long long)b << 4) | (unsigned)j;
    }
  }
  if (bad) flag_status(a.status, kBadConf);
  for (int i = nk + tid; i < M; i += kThreads) keys[i] = ~0ull;
  if (tid == 0) first_fail = nk;
  for (int b = tid; b < B; b += kThreads) a.budget[b] = 0;
  __threadfence();
  __syncthreads();

  for (int k = 2; k <= M; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < M; i += kThreads) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const unsigned long long x = keys[i], y = keys[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) keys[i] = y, keys[ixj] = x;
        }
      }
      __syncthreads();
    }
  }

  // thread tid owns sorted candidates [lo, hi)
  const int per = (nk + kThreads - 1) / kThreads;
  const int lo = min(tid * per, nk), hi = min(lo + per, nk);
  unsigned long long local = 0;
  for (int i = lo; i < hi; ++i) local += 0xFFFFFFFFull - (keys[i] >> 32);
  part[tid] = local;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {  // inclusive scan of the thread sums
    const unsigned long long v = tid >= o ? part[tid - o] : 0ull;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  unsigned long long tau = ((unsigned long long)B << 32) + part[tid] - local;
  for (int i = lo; i < hi; ++i) {
    const unsigned long long q = 0xFFFFFFFFull - (keys[i] >> 32);
    const double N = (double)(B + i);
    const double lhs = (double)(tau + q) * step_time(N, tB, tT, np);
    const double rhs = (double)tau * step_time(N + 1.0, tB, tT, np);
    if (!(lhs > rhs)) {
      atomicMin(&first_fail, i);
      break;
    }
    tau += q;
  }
  __syncthreads();
  const int stop = first_fail;
  for (int i = tid; i < stop; i += kThreads) {
    const int b = (int)((keys[i] >> 4) & 0x0FFFFFFFull);
    atomicAdd(&a.budget[b], 1);
  }
}

}  // namespace

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
  schedule_kernel<<<1, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dspark

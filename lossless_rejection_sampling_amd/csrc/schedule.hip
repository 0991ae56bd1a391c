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

#pragma clang fp contract(off)

// 1/SPS at a verify batch of N tokens (see the ABI header for the rule).
__device__ double step_time(double N, const double* Bs, const double* sv, int np) {
  if (N <= Bs[0]) return 1.0 / sv[0];
  int i = 0;
  while (i + 1 < np - 1 && Bs[i + 1] <= N) ++i;
  const double t0 = 1.0 / sv[i], t1 = 1.0 / sv[i + 1];
  const double frac = (N - Bs[i]) / (Bs[i + 1] - Bs[i]);
  const double dt = t1 - t0;
  const double inc = dt * frac;
  return t0 + inc;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(ScheduleArgs a) {
  __shared__ unsigned long long keys[kMaxKeys];
  __shared__ unsigned long long part[kThreads];
  __shared__ int first_fail;
  const int tid = threadIdx.x, B = a.B, gamma = a.gamma;
  const int nk = B * gamma;
  int M = 1;
  while (M < nk) M <<= 1;

  for (int b = tid; b < B; b += kThreads) {
    float acc = 1.0f;
    for (int j = 0; j < gamma; ++j) {
      float c = a.conf[(size_t)b * gamma + j];
      if (!(c > 0.0f && c < 1.0f)) {
        flag_status(a.status, kBadConf);
        c = c > 0.0f ? 0x1.fffffep-1f : 0x1p-126f;  // clamp into (0, 1); NaN -> tiny
      }
      acc = acc * c;
      const unsigned long long q = (unsigned long long)floor((double)acc * 4294967296.0);
      keys[b * gamma + j] = ((0xFFFFFFFFull - q) << 32) | ((unsigned long long)b << 4) | (unsigned)j;
    }
  }
  for (int i = nk + tid; i < M; i += kThreads) keys[i] = ~0ull;
  if (tid == 0) first_fail = nk;
  for (int b = tid; b < B; b += kThreads) a.budget[b] = 0;
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
    const double lhs = (double)(tau + q) * step_time(N, a.sps_B, a.sps_val, a.n_points);
    const double rhs = (double)tau * step_time(N + 1.0, a.sps_B, a.sps_val, a.n_points);
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

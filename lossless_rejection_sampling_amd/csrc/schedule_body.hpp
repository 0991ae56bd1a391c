// Body of the hardware-aware prefix scheduler, shared by its own launch and by
// the launch that runs it beside the last draft draw (see schedule.hip for the
// method).  Everything here has internal linkage in each including file.
#pragma once
#include <math.h>

#include "dspark.h"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerCand = 16;
constexpr int kCandPerGroup = kThreads / kLanesPerCand;
constexpr uint32_t kNoFail = 0x7fffffffu;
constexpr int kMaxGamma = 16;  // the ABI's largest block length

// 1/SPS at a verify batch of N tokens (see the ABI header for the rule), from
// the table in LDS: batch sizes Bs and step times ts = 1/SPS.  The segment is
// the last i <= np-2 with Bs[i] <= N (binary search).
__device__ __forceinline__ double step_time(double N, const double* Bs, const double* ts, int np) {
#pragma clang fp contract(off)
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

// Sequential Temperature Scaling of one score: 1 / (1 + exp(-z / tau)),
// z = ln c - ln(1 - c), in fp64 from the fp32 score, rounded once to fp32 and
// kept strictly inside (0, 1).
__device__ __forceinline__ float scaled_score(float c, float tau) {
#pragma clang fp contract(off)
  const double x = (double)c;
  const double z = log(x) - log1p(-x);
  double y = 1.0 / (1.0 + exp(-z / (double)tau));
  y = fmin(fmax(y, 0x1p-126), 0x1.fffffep-1);
  return (float)y;
}

__device__ __forceinline__ void store_coherent(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), (unsigned long long)__double_as_longlong(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_coherent(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<double*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// One workgroup (index bid of nblocks) of the scheduler; smem: dynamic LDS of
// schedule_lds_bytes().  Every workgroup of the launch runs this.
__device__ __forceinline__ void schedule_block(const ScheduleArgs& a, int bid, int nblocks, char* smem) {
#pragma clang fp contract(off)
  __shared__ int s_last;
  __shared__ double s_best[kThreads / 64];
  __shared__ int s_bestm[kThreads / 64];
  const int tid = threadIdx.x, B = a.B, gamma = a.gamma, np = a.n_points;
  const int nk = B * gamma;
  // key of candidate m = b * gamma + j: (0xFFFFFFFF - Q) 2^32 + m, ascending in the admission order
  unsigned long long* const key = reinterpret_cast<unsigned long long*>(smem);
  double* const tB = reinterpret_cast<double*>(smem + (size_t)((nk + 1) & ~1) * 8);
  double* const tT = tB + np;
  const bool ranked = a.rule == DSPARK_SCHED_EARLY_STOP || a.rule == DSPARK_SCHED_ARGMAX;

  // the table: batch sizes strictly increasing, rates positive and finite (else
  // a status bit; the budgets are then unspecified, every access stays in bounds)
  bool bad_table = false;
  for (int i = tid; i < np; i += kThreads) {
    const double bi = a.sps_B[i], vi = a.sps_val[i];
    tB[i] = bi;
    tT[i] = 1.0 / vi;
    if (!(vi > 0.0 && vi < INFINITY) || !(bi < INFINITY) || (i > 0 && !(bi > a.sps_B[i - 1]))) bad_table = true;
  }
  if (bad_table && bid == 0) flag_status(a.status, kBadTable);
  bool bad = false;
  const float thr = (float)a.param;
  for (int b = tid; b < B; b += kThreads) {
    float acc = 1.0f;
    int lead = 0;  // leading positions above the threshold
    bool run = true;
    auto admit = [&](int j, float cj) {
      if (!(cj > 0.0f && cj < 1.0f)) {
        bad = true;
        cj = cj > 0.0f ? 0x1.fffffep-1f : 0x1p-126f;  // clamp into (0, 1); NaN -> tiny
      }
      if (a.tau) cj = scaled_score(cj, a.tau[j]);
      run = run && cj > thr;
      lead += run ? 1 : 0;
      acc = acc * cj;
      const uint32_t q = (uint32_t)floor((double)acc * 4294967296.0);
      key[b * gamma + j] = ((unsigned long long)(0xFFFFFFFFu - q) << 32) | (uint32_t)(b * gamma + j);
    };
    if (!a.tau) {
      // the request's scores in one memory round trip (gamma <= kMaxGamma)
      float cv[kMaxGamma];
#pragma unroll
      for (int j = 0; j < kMaxGamma; ++j) cv[j] = j < gamma ? a.conf[(size_t)b * gamma + j] : 0.5f;
#pragma unroll
      for (int j = 0; j < kMaxGamma; ++j)
        if (j < gamma) admit(j, cv[j]);
    } else {
      for (int j = 0; j < gamma; ++j) admit(j, a.conf[(size_t)b * gamma + j]);
    }
    if (bid == 0 && !ranked) {
      const int fixed = (int)fmin(fmax(a.param, 0.0), (double)gamma);
      a.budget[b] = a.rule == DSPARK_SCHED_FIXED ? fixed : lead;
    }
  }
  // padding to a whole 16-byte word: a key after every candidate's, which no candidate counts
  if (tid == 0 && (nk & 1)) key[nk] = ~0ull;
  if (bad && bid == 0) flag_status(a.status, kBadConf);
  if (!ranked) return;  // uniform: the fixed and threshold rules are done
  __syncthreads();

  // candidate i: keys before it and the sum of their Q; lane `sub` reads keys
  // 2 (sub + 16 t) and the next as one 16-byte word (the padding key never counts)
  const int i = bid * kCandPerGroup + (tid / kLanesPerCand), sub = tid % kLanesPerCand;
  uint32_t cnt = 0;
  unsigned long long tau = 0;
  const unsigned long long ki = i < nk ? key[i] : 0ull;
  const uint32_t qi = (uint32_t)(ki >> 32);
  if (i < nk) {
    const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(key);
    const int n2 = (nk + 1) / 2;
    auto count = [&](const ulonglong2& w) {
      const bool b0 = w.x < ki, b1 = w.y < ki;
      cnt += (b0 ? 1u : 0u) + (b1 ? 1u : 0u);
      tau += (b0 ? 0xFFFFFFFFull - (w.x >> 32) : 0ull) + (b1 ? 0xFFFFFFFFull - (w.y >> 32) : 0ull);
    };
    // eight LDS reads in flight per lane
    int t = sub;
    for (; t + 7 * kLanesPerCand < n2; t += 8 * kLanesPerCand) {
      ulonglong2 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = k2[t + u * kLanesPerCand];
#pragma unroll
      for (int u = 0; u < 8; ++u) count(w[u]);
    }
    for (; t < n2; t += kLanesPerCand) count(k2[t]);
  }
  static_assert(kLanesPerCand == 16, "one DPP row per candidate");
  cnt = reduce16(cnt, OpSum{});
  tau = reduce16(tau, OpSum{});
  if (i < nk && sub == 0) {
    const unsigned long long q = 0xFFFFFFFFull - qi;
    const unsigned long long T = ((unsigned long long)B << 32) + tau;
    const double N = (double)(B + (int)cnt);
    if (a.rule == DSPARK_SCHED_EARLY_STOP) {
      const double lhs = (double)(T + q) * step_time(N, tB, tT, np);
      const double rhs = (double)T * step_time(N + 1.0, tB, tT, np);
      if (!(lhs > rhs)) atomicMax(a.stop_enc, kNoFail - cnt);
    } else {
      store_coherent(a.theta + cnt + 1, (double)(T + q) / step_time(N + 1.0, tB, tT, np));
    }
    __hip_atomic_store(a.rank + i, (int)cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (a.rule == DSPARK_SCHED_ARGMAX && bid == 0 && tid == 0)
    store_coherent(a.theta, (double)((unsigned long long)B << 32) / step_time((double)B, tB, tT, np));

  // The last workgroup to finish turns ranks into budgets.  Ranks and Theta
  // travel as agent-scope atomics (coherent across the XCDs' L2 caches without
  // a cache-wide writeback or invalidate): every wavefront waits for its own
  // stores to complete before the barrier, and the ticket is taken after it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  asm volatile(";; dspark publish: scheduler ticket" ::: "memory");  // a comment: no instruction
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nblocks - 1);
  __syncthreads();
  if (!s_last) return;
  // the ranks of this thread's first request, requested with the cut's inputs
  int rk[kMaxGamma];
  auto load_ranks = [&](int b) {
#pragma unroll
    for (int j = 0; j < kMaxGamma; ++j)
      rk[j] = j < gamma ? __hip_atomic_load(a.rank + b * gamma + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  };
  if (tid < B) load_ranks(tid);
  int stop;
  if (a.rule == DSPARK_SCHED_EARLY_STOP) {
    const uint32_t enc = __hip_atomic_load(a.stop_enc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stop = enc ? (int)(kNoFail - enc) : nk;
  } else {
    // the first largest Theta over the cuts m = 0..nk, 8 loads in flight a thread
    double best = -1.0;
    int bm = 0x7fffffff;
    for (int m0 = tid; m0 <= nk; m0 += 8 * kThreads) {
      double th[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) th[u] = m0 + u * kThreads <= nk ? load_coherent(a.theta + m0 + u * kThreads) : -1.0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (th[u] > best) best = th[u], bm = m0 + u * kThreads;  // m increases: ties keep the first
    }
    wave_argmax(best, bm);
    if ((tid & 63) == 0) s_best[tid >> 6] = best, s_bestm[tid >> 6] = bm;
    __syncthreads();
    best = -1.0, bm = 0x7fffffff;
    for (int w = 0; w < kThreads / 64; ++w)
      if (s_best[w] > best || (s_best[w] == best && s_bestm[w] < bm)) best = s_best[w], bm = s_bestm[w];
    stop = index_or(bm, nk + 1, 0);
  }
  for (int b = tid; b < B; b += kThreads) {
    if (b != tid) load_ranks(b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < kMaxGamma; ++j) n += j < gamma && rk[j] < stop ? 1 : 0;
    a.budget[b] = n;
  }
  if (tid == 0) {
    __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.stop_enc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace
}  // namespace dspark

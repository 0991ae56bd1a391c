// Verify half of the round: lossless rejection sampling of the drafted block.
//
// Each draft token x_k is accepted with probability min(1, p_k(x_k) / q_k(x_k));
// verification stops at the first rejection, whose token is redrawn from the
// residual distribution, and a fully accepted block earns a bonus token from the
// target ("Les mathématiques derrière l'accélération ...", section "La garantie
// de l'échantillonnage par rejet"; "DeepSeek发布DSpark", section "DSpark 是什么？").
// The residual is max(0, p - q) normalised.
//
// Kernels, in launch order:
//   verify_prep       clear the residual work list, check budgets
//   row_stats         one wavefront per (target row, 4096-column block): max,
//                     exp-sum relative to the max, argmax      [HBM-bound pass]
//   accept            one wavefront per request: accept tests, bonus draw or
//                     greedy argmax, queue of requests that rejected
//   (gemm_stats)      residual mass of every tile of the rejected rows
//   residual_select   one wavefront per rejected request: draw from the residual
//   residual_debug    optional: the normalised residual row
#include <math.h>

#include "dspark.h"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int budget_of(const VerifyArgs& a, int b) {
  if (!a.budget) return a.gamma;
  const int L = a.budget[b];
  return L < 0 ? 0 : (L > a.gamma ? a.gamma : L);
}

__global__ void verify_prep_kernel(VerifyArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b == 0) *a.slot_count = 0u;
  if (b < a.B) {
    a.req[b].pending = 0;
    if (a.budget && (a.budget[b] < 0 || a.budget[b] > a.gamma)) flag_status(a.status, kBadBudget);
  }
}

// ---------------------------------------------------------------------------
// Target row statistics.  A lane holds 64 logits of the block in registers:
// vector path, bf16: element i*512 + lane*8 + q (eight 16-byte loads);
// vector path, fp32: element i*256 + lane*4 + q (sixteen 16-byte loads);
// scalar path: element i*64 + lane.
// ---------------------------------------------------------------------------
template <typename TL, bool VEC>
__global__ __launch_bounds__(64) void row_stats_kernel(VerifyArgs a) {
  const int blk = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
  const int gamma = a.gamma, V = a.V;
  const int b = row / (gamma + 1), j = row - b * (gamma + 1);
  if (j > budget_of(a, b)) return;
  const float T = effective_temp(a.temperature[b]);
  const int start = blk * kBlock;
  const int len = min(kBlock, V - start);
  const TL* p = static_cast<const TL*>(a.target) + (size_t)row * V + start;

  float z[64];
  int idx0, stride_i, per;  // element of register (i, q) = idx0 + i*stride_i + q, q < per
  if (VEC && len == kBlock) {
    if constexpr (sizeof(TL) == 2) {
      idx0 = lane * 8, stride_i = 512, per = 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(p + idx0 + i * 512);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[i * 8 + 2 * q] = __uint_as_float(ww[q] << 16);
          z[i * 8 + 2 * q + 1] = __uint_as_float(ww[q] & 0xffff0000u);
        }
      }
    } else {
      idx0 = lane * 4, stride_i = 256, per = 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 w = *reinterpret_cast<const float4*>(p + idx0 + i * 256);
        z[i * 4] = w.x, z[i * 4 + 1] = w.y, z[i * 4 + 2] = w.z, z[i * 4 + 3] = w.w;
      }
    }
  } else {
    idx0 = lane, stride_i = 64, per = 1;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int e = i * 64 + lane;
      z[i] = e < len ? load_logit(p + e) : -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 64; ++i) m = fmaxf(m, z[i]);
  m = wave_max(m);
  float s = 0.0f;
  int arg = 0x7fffffff;
  if (T > 0.0f) {
    const float c = kLog2e / T;
#pragma unroll
    for (int i = 0; i < 64; ++i) s += exp2f((z[i] - m) * c);
    s = wave_sum(s);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int e = idx0 + (i / per) * stride_i + (i % per);
      if (z[i] == m && e < arg) arg = e;
    }
    arg = wave_min_int(arg);
  }
  if (lane == 0) {
    BlockStat st;
    st.mx = m, st.sum = s, st.arg = arg == 0x7fffffff ? -1 : start + arg, st.pad = 0.0f;
    a.bstat[(size_t)row * a.n_blk + blk] = st;
  }
}

// ln-sum-exp of one target row from its block statistics: row maximum M and
// ln sum_v exp((z_v - M) / T).
__device__ __forceinline__ void row_lse(const BlockStat* bs, int nb, double invT, int lane, double& M,
                                        double& logsum) {
  double m = -INFINITY;
  for (int i = lane; i < nb; i += 64) m = fmax(m, (double)bs[i].mx);
  M = wave_max(m);
  double s = 0.0;
  for (int i = lane; i < nb; i += 64) s += (double)bs[i].sum * exp(((double)bs[i].mx - M) * invT);
  logsum = log(wave_sum(s));
}

// Lowest index of the row maximum.
__device__ __forceinline__ int row_argmax(const BlockStat* bs, int nb, int lane) {
  double best = -INFINITY;
  int arg = 0x7fffffff;
  for (int i = lane; i < nb; i += 64) {
    const double m = bs[i].mx;
    if (m > best || (m == best && bs[i].arg < arg)) best = m, arg = bs[i].arg;
  }
  wave_argmax(best, arg);
  return arg;
}

// Three-level Gumbel-max draw from softmax(row / T): block from the block
// statistics, tile from the chosen block (reread), column from the chosen tile.
template <typename TL>
__device__ int sample_row(const TL* row, const BlockStat* bs, int nb, int V, double invT,
                          uint64_t seed, uint32_t req, uint32_t rpos, int lane) {
  const double mref = bs[0].mx;
  double best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = lane; i < nb; i += 64) {
    const double val = ((double)bs[i].mx - mref) * invT + log((double)bs[i].sum) +
                       gumbel(seed, kFinalTop, req, rpos, i);
    if (val > best) best = val, bi = i;
  }
  wave_argmax(best, bi);
  bi = index_or(bi, nb, 0);

  const int start = bi * kBlock, len = min(kBlock, V - start);
  double val = -INFINITY;
  int ti = 0x7fffffff;
  if (lane * kTile < len) {
    const TL* tp = row + start + lane * kTile;
    const int tl = min(kTile, len - lane * kTile);
    float mt = -INFINITY;
    for (int e = 0; e < tl; ++e) mt = fmaxf(mt, load_logit(tp + e));
    double st = 0.0;
    for (int e = 0; e < tl; ++e) st += exp(((double)load_logit(tp + e) - (double)mt) * invT);
    val = ((double)mt - mref) * invT + log(st) + gumbel(seed, kFinalMid, req, rpos, lane);
    ti = lane;
  }
  wave_argmax(val, ti);
  ti = index_or(ti, (len + kTile - 1) / kTile, 0);

  const int tstart = start + ti * kTile;
  double lv = -INFINITY;
  int vi = 0x7fffffff;
  if (tstart + lane < min(start + len, tstart + kTile)) {
    lv = (double)load_logit(row + tstart + lane) * invT + gumbel(seed, kFinalLeaf, req, rpos, lane);
    vi = tstart + lane;
  }
  wave_argmax(lv, vi);
  return index_or(vi, min(start + len, tstart + kTile), tstart);
}

template <typename TL>
__global__ __launch_bounds__(64) void accept_kernel(VerifyArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int gamma = a.gamma, V = a.V, nb = a.n_blk;
  const int L = budget_of(a, b);
  const float Tf = checked_temp(a.temperature[b], a.status);
  const bool greedy = !(Tf > 0.0f);
  const double invT = greedy ? 0.0 : 1.0 / (double)Tf;
  const uint32_t off = a.pos_offset ? (uint32_t)a.pos_offset[b] : 0u;
  const BlockStat* bs = a.bstat + (size_t)b * (gamma + 1) * nb;
  const TL* trow0 = static_cast<const TL*>(a.target) + (size_t)b * (gamma + 1) * V;
  const int32_t* xs = a.draft + (size_t)b * gamma;

  int n = 0;
  for (int k = 1; k <= L; ++k) {
    const int j = k - 1;
    const int x = checked_token(xs[j], V, a.status, kBadDraft);
    bool ok;
    if (greedy) {
      ok = x == row_argmax(bs + (size_t)j * nb, nb, lane);
    } else {
      double M, lS;
      row_lse(bs + (size_t)j * nb, nb, invT, lane, M, lS);
      const double lp = ((double)load_logit(trow0 + (size_t)j * V + x) - M) * invT - lS;
      const double lq = (double)a.draft_logq[(size_t)b * gamma + j];
      const double lnu = log(uniform_from_word(rng_word(a.seed, kAccept, b, k + off, 0)));
      ok = lnu < lp - lq;  // u < min(1, p/q) since ln u < 0
      if (a.debug_logp_logq && lane == 0) {
        a.debug_logp_logq[((size_t)b * gamma + j) * 2] = (float)lp;
        a.debug_logp_logq[((size_t)b * gamma + j) * 2 + 1] = (float)lq;
      }
    }
    if (!ok) break;
    ++n;
  }

  int y = -1;
  const BlockStat* bn = bs + (size_t)n * nb;
  if (greedy) {
    y = row_argmax(bn, nb, lane);
  } else if (n == L) {
    y = sample_row(trow0 + (size_t)n * V, bn, nb, V, invT, a.seed, b, n + 1 + off, lane);
  } else {
    double M, lS;
    row_lse(bn, nb, invT, lane, M, lS);
    if (lane == 0) {
      ReqState st;
      st.row_max = M, st.row_logsum = lS, st.res_mass = 0.0, st.n = n, st.pending = 1;
      a.req[b] = st;
      a.slot_req[atomicAdd(a.slot_count, 1u)] = b;
    }
  }
  for (int i = lane; i <= gamma; i += 64) {
    int t = -1;
    if (i < n) t = xs[i];
    else if (i == n) t = y;
    a.out_tokens[(size_t)b * (gamma + 1) + i] = t;
  }
  if (lane == 0) {
    a.num_accepted[b] = n;
    a.num_emitted[b] = n + 1;
  }
}

// fp64 residual r(v) = max(0, p(v) - q(v)) at one column of the rejected row.
template <typename TL, typename TF>
__device__ __forceinline__ double residual_at(const VerifyArgs& a, int b, const ReqState& st,
                                              int prev, double invT, double lse_q, int v,
                                              double* p_out) {
  const int V = a.V, r = a.r, n = st.n;
  const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (a.gamma + 1) + n) * V;
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * a.gamma + n) * V;
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  const TF* w = static_cast<const TF*>(a.Wt) + (size_t)v * r;
  double acc = 0.0;
  for (int k = 0; k < r; ++k) acc += (double)load_logit(h + k) * (double)load_logit(w + k);
  const double d = (double)load_logit(brow + v) + acc;
  const double p = exp(((double)load_logit(trow + v) - st.row_max) * invT - st.row_logsum);
  const double q = exp(d * invT - lse_q);
  if (p_out) *p_out = p;
  return p > q ? p - q : 0.0;
}

template <typename TL, typename TF>
__global__ __launch_bounds__(64) void residual_select_kernel(VerifyArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const ReqState st = a.req[b];
  if (!st.pending) return;
  const int gamma = a.gamma, V = a.V, nt = a.n_tiles, n = st.n;
  const double invT = 1.0 / (double)a.temperature[b];
  const uint32_t off = a.pos_offset ? (uint32_t)a.pos_offset[b] : 0u;
  const uint32_t rpos = n + 1 + off;
  int prev = n == 0 ? a.prev0[b] : a.draft[(size_t)b * gamma + n - 1];
  prev = checked_token(prev, V, a.status, n == 0 ? kBadPrev : kBadDraft);
  const double lse_q = a.draft_lse[(size_t)b * gamma + n];
  const float* R = a.rsum + (size_t)b * nt;
  const int nblk = (nt + kTilesPerBlock - 1) / kTilesPerBlock;

  double tot = 0.0, best = -INFINITY;
  int bi = 0x7fffffff;
  for (int blk = lane; blk < nblk; blk += 64) {
    double rb = 0.0;
    for (int t = blk * kTilesPerBlock; t < min((blk + 1) * kTilesPerBlock, nt); ++t) rb += (double)R[t];
    tot += rb;
    if (rb > 0.0) {
      const double val = log(rb) + gumbel(a.seed, kFinalTop, b, rpos, blk);
      if (val > best) best = val, bi = blk;
    }
  }
  tot = wave_sum(tot);
  wave_argmax(best, bi);

  int y;
  const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (gamma + 1) + n) * V;
  if (!(tot > 0.0)) {
    // no residual mass: draw from p itself
    y = sample_row(trow, a.bstat + ((size_t)b * (gamma + 1) + n) * a.n_blk, a.n_blk, V, invT, a.seed,
                   b, rpos, lane);
  } else {
    bi = index_or(bi, nblk, 0);
    const int t0 = bi * kTilesPerBlock, t1 = min(t0 + kTilesPerBlock, nt);
    double val = -INFINITY;
    int ti = 0x7fffffff;
    if (t0 + lane < t1 && R[t0 + lane] > 0.0f) {
      val = log((double)R[t0 + lane]) + gumbel(a.seed, kFinalMid, b, rpos, lane);
      ti = t0 + lane;
    }
    wave_argmax(val, ti);
    ti = index_or(ti, t1, t0);
    const int v = ti * kTile + lane;
    double lv = -INFINITY, lp = -INFINITY;
    int vi = 0x7fffffff;
    if (v < V) {
      double p;
      const double rv = residual_at<TL, TF>(a, b, st, prev, invT, lse_q, v, &p);
      const double g = gumbel(a.seed, kFinalLeaf, b, rpos, lane);
      if (rv > 0.0) lv = log(rv) + g, vi = v;
      lp = log(p) + g;
    }
    wave_argmax(lv, vi);
    if (vi == 0x7fffffff) {  // the chosen tile lost all residual mass in fp64
      vi = v < V ? v : 0x7fffffff;
      wave_argmax(lp, vi);
    }
    y = index_or(vi, min(V, (ti + 1) * kTile), ti * kTile);
  }
  if (lane == 0) {
    a.out_tokens[(size_t)b * (gamma + 1) + n] = y;
    a.req[b].res_mass = tot;
  }
}

template <typename TL, typename TF>
__global__ __launch_bounds__(64) void residual_debug_kernel(VerifyArgs a) {
  const int tile = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const ReqState st = a.req[b];
  if (!st.pending) return;
  const int v = tile * kTile + lane;
  if (v >= a.V) return;
  const int gamma = a.gamma, n = st.n;
  int prev = n == 0 ? a.prev0[b] : a.draft[(size_t)b * gamma + n - 1];
  prev = prev < 0 ? 0 : (prev >= a.V ? a.V - 1 : prev);
  const double invT = 1.0 / (double)a.temperature[b];
  double p;
  const double rv = residual_at<TL, TF>(a, b, st, prev, invT, a.draft_lse[(size_t)b * gamma + n], v, &p);
  a.debug_residual[(size_t)b * a.V + v] = (float)(st.res_mass > 0.0 ? rv / st.res_mass : p);
}

}  // namespace

hipError_t launch_verify_prep(const VerifyArgs& a, hipStream_t s) {
  verify_prep_kernel<<<(a.B + 255) / 256, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_row_stats(const VerifyArgs& a, int logits_dtype, hipStream_t s) {
  const dim3 grid(a.n_blk, a.B * (a.gamma + 1));
  if (logits_dtype == DSPARK_BF16) {
    if (a.V % 8 == 0) row_stats_kernel<uint16_t, true><<<grid, 64, 0, s>>>(a);
    else row_stats_kernel<uint16_t, false><<<grid, 64, 0, s>>>(a);
  } else {
    if (a.V % 4 == 0) row_stats_kernel<float, true><<<grid, 64, 0, s>>>(a);
    else row_stats_kernel<float, false><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_accept(const VerifyArgs& a, int logits_dtype, hipStream_t s) {
  if (logits_dtype == DSPARK_BF16) accept_kernel<uint16_t><<<a.B, 64, 0, s>>>(a);
  else accept_kernel<float><<<a.B, 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_residual_select(const VerifyArgs& a, int logits_dtype, int factor_dtype,
                                  hipStream_t s) {
  if (logits_dtype == DSPARK_BF16) {
    if (factor_dtype == DSPARK_BF16) residual_select_kernel<uint16_t, uint16_t><<<a.B, 64, 0, s>>>(a);
    else residual_select_kernel<uint16_t, float><<<a.B, 64, 0, s>>>(a);
  } else {
    if (factor_dtype == DSPARK_BF16) residual_select_kernel<float, uint16_t><<<a.B, 64, 0, s>>>(a);
    else residual_select_kernel<float, float><<<a.B, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_residual_debug(const VerifyArgs& a, int logits_dtype, int factor_dtype,
                                 hipStream_t s) {
  const dim3 grid(a.n_tiles, a.B);
  if (logits_dtype == DSPARK_BF16) {
    if (factor_dtype == DSPARK_BF16) residual_debug_kernel<uint16_t, uint16_t><<<grid, 64, 0, s>>>(a);
    else residual_debug_kernel<uint16_t, float><<<grid, 64, 0, s>>>(a);
  } else {
    if (factor_dtype == DSPARK_BF16) residual_debug_kernel<float, uint16_t><<<grid, 64, 0, s>>>(a);
    else residual_debug_kernel<float, float><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dspark

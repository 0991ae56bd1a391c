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
//   verify_lazy       one workgroup per (target row, request, 4 consecutive
//                     4096-column blocks), position-major: max, exp-sum relative to the
//                     max, argmax of the rows still needed [HBM-bound pass];
//                     the accept tests run as rows complete; the wavefront
//                     that decides a request emits its accepted tokens and
//                     counts, and its greedy final token
//   (gemm_stats)      residual mass of every tile of the rejected rows
//   residual_select   one workgroup per request still drawing: a draw from the
//                     residual of a rejected row, or the bonus from target row L;
//                     every workgroup first zeroes its request's counters of the
//                     lazy pass (and workgroup 0 the residual work list), so a
//                     call leaves them as the next one needs them
//   residual_debug    optional: the normalised residual row
// row_stats (the same statistics for every row 0..L_b) serves the analytic
// acceptance pass.
#include <math.h>

#include "dspark.h"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int budget_of(const VerifyArgs& a, int b) {
  if (!a.budget) return a.gamma;
  const int L = a.budget[b];
  return L < 0 ? 0 : (L > a.gamma ? a.gamma : L);
}


// v_exp_f32 itself: results below 2^-126 flush to zero.  A block sum taken
// relative to the block maximum holds a term of 1, so the flushed terms cannot
// change it; exp2f spends five more instructions per element keeping them.
__device__ __forceinline__ float exp2_flush(float x) { return __builtin_amdgcn_exp2f(x); }

// max of three: fmaxf would first quiet (canonicalise) each value made by bit
// operations, one more instruction per element
__device__ __forceinline__ float max3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

// ---------------------------------------------------------------------------
// Target row statistics.  A lane holds 64 logits of the block in registers:
// vector path, bf16: element i*512 + lane*8 + q (eight 16-byte loads);
// vector path, fp32: element i*256 + lane*4 + q (sixteen 16-byte loads);
// scalar path: element i*64 + lane.
// ---------------------------------------------------------------------------
template <typename TL, bool VEC>
__device__ __forceinline__ BlockStat block_stats(const VerifyArgs& a, int row, int blk, float T, int lane) {
  const int V = a.V;
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
        // streaming loads: every target row is read once, and W2 (read again by the
        // residual pass) stays in the Infinity Cache
        const u32x4n w = __builtin_nontemporal_load(reinterpret_cast<const u32x4n*>(p + idx0 + i * 512));
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
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 64; i += 4) m0 = max3(m0, z[i], z[i + 1]), m1 = max3(m1, z[i + 2], z[i + 3]);
  const float m = wave_max(fmaxf(m0, m1));
  float s = 0.0f;
  int arg = 0x7fffffff;
  if (T > 0.0f) {
    // 2^((z - m) c): the difference first (exact for bf16 inputs, one rounding
    // relative to |z - m| for fp32), so the terms near the maximum carry no
    // error proportional to |m| / T, as a shift by a rounded m c would
    const float c = kLog2e / T, mm = m == -INFINITY ? 0.0f : m;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; i += 2) s0 += exp2_flush((z[i] - mm) * c), s1 += exp2_flush((z[i + 1] - mm) * c);
    s = wave_sum(s0 + s1);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int e = idx0 + (i / per) * stride_i + (i % per);
      if (z[i] == m && e < arg) arg = e;
    }
    arg = wave_min_int(arg);
  }
  BlockStat st;
  st.mx = m, st.sum = s, st.arg = arg == 0x7fffffff ? -1 : start + arg, st.pad = 0.0f;
  return st;
}

template <typename TL, bool VEC>
__global__ __launch_bounds__(64) void row_stats_kernel(VerifyArgs a) {
  const int blk = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
  const int gamma = a.gamma;
  // the accept pass appends to the residual work list after this kernel
  if (blk == 0 && row == 0 && lane == 0) *a.slot_count = 0u;
  const int b = row / (gamma + 1), j = row - b * (gamma + 1);
  if (j > budget_of(a, b)) return;
  const BlockStat st = block_stats<TL, VEC>(a, row, blk, effective_temp(a.temperature[b]), lane);
  if (lane == 0) a.bstat[(size_t)row * a.n_blk + blk] = st;
}

// Block statistics exchanged between the workgroups of one pass (lazy
// verification): written and read as agent-scope atomics (coherent across the
// XCDs' L2 caches, with no cache-wide writeback or invalidate), 8 bytes at a time.
__device__ __forceinline__ void store_bstat_coherent(BlockStat* p, const BlockStat& st) {
  uint64_t w[2];
  __builtin_memcpy(w, &st, sizeof(w));
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ BlockStat load_bstat_coherent(const BlockStat* p) {
  uint64_t w[2];
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<BlockStat*>(p));
  w[0] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  w[1] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  BlockStat st;
  __builtin_memcpy(&st, w, sizeof(w));
  return st;
}

// Statistics of target rows 0..nrows-1 of one request from their block
// statistics, one wavefront per row: maximum M, ln sum_v exp((z_v - M) / T)
// and, for greedy requests, the lowest index of the maximum.
struct RowInfo {
  double M, logS;
  int arg;
};

__device__ __forceinline__ RowInfo row_info(const BlockStat* bs, int nb, bool greedy, double invT, int lane) {
  RowInfo ri;
  double m = -INFINITY;
  int arg = 0x7fffffff;
  for (int i = lane; i < nb; i += 64) {
    const BlockStat st = load_bstat_coherent(bs + i);
    const double mi = st.mx;
    if (mi > m || (greedy && mi == m && st.arg < arg)) m = mi, arg = st.arg;
  }
  double mm = m;
  int aa = arg;
  wave_argmax(mm, aa);
  ri.M = mm;
  ri.arg = aa;
  ri.logS = 0.0;
  if (!greedy) {
    double sum = 0.0;
    for (int i = lane; i < nb; i += 64) {
      const BlockStat st = load_bstat_coherent(bs + i);
      sum += (double)st.sum * exp(((double)st.mx - mm) * invT);
    }
    ri.logS = log(wave_sum(sum));
  }
  return ri;
}

// Three-level Gumbel-max draw from softmax(row / T) by wavefront 0 of the
// workgroup: block from the block statistics, tile from a re-read of the chosen
// block (one 64-column tile per lane), column from the chosen tile.
template <typename TL>
__device__ int sample_row(const TL* row, const BlockStat* bs, int nb, int V, double invT, uint64_t seed,
                          uint32_t req, uint32_t rpos, int lane) {
  const double mref = load_bstat_coherent(bs).mx;
  double best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = lane; i < nb; i += 64) {
    const BlockStat st = load_bstat_coherent(bs + i);
    const double val = ((double)st.mx - mref) * invT + log((double)st.sum) + gumbel(seed, kFinalTop, req, rpos, i);
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
    float z[kTile];
    const bool vec = tl == kTile && (reinterpret_cast<uintptr_t>(tp) & 15) == 0;
    if (vec) {
      if constexpr (sizeof(TL) == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 w = reinterpret_cast<const uint4*>(tp)[i];
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            z[8 * i + 2 * q] = __uint_as_float(ww[q] << 16);
            z[8 * i + 2 * q + 1] = __uint_as_float(ww[q] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float4 w = reinterpret_cast<const float4*>(tp)[i];
          z[4 * i] = w.x, z[4 * i + 1] = w.y, z[4 * i + 2] = w.z, z[4 * i + 3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < kTile; ++e) z[e] = e < tl ? load_logit(tp + e) : -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < kTile; ++e) mt = fmaxf(mt, z[e]);
    const float c = (float)invT;
    float st = 0.0f;
#pragma unroll
    for (int e = 0; e < kTile; ++e) st += expf((z[e] - mt) * c);
    val = ((double)mt - mref) * invT + log((double)st) + gumbel(seed, kFinalMid, req, rpos, lane);
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

// ---------------------------------------------------------------------------
// Lazy verification: a target row from row 2 on is skipped once its request is
// known to be decided, so the rows read are 0..max(n_b, 1) plus the few read
// before the decision was known (instead of 0..L_b).  One workgroup of 4 wavefronts per work item
// (target row j, request b, 4 consecutive 4096-column blocks, one per
// wavefront) in position-major order,
//   item = (j B + b) ceil(n_blk / 4) + chunk,
// so the rows of early positions, whose tests decide which later rows are
// needed, are read first.  No item waits for another.
//
// Progress of request b, one word changed only by atomic read-modify-writes:
//   bit j (j <= 16)   target row j has all its block statistics
//   bits 20..24       m: positions 1..m tested and accepted
//   bit 31            the final token is decided (no further row is needed)
// The test of position j + 1 needs row j complete and m = j.  The last block of
// row j sets bit j and runs the test if it finds m = j; the wavefront that
// raises m to j runs it if it finds bit j set; each read-modify-write sees the
// other's, so exactly one of them runs it.  A tester goes on with the next
// position while the next row is already complete.  The final token: a failed
// test at position n + 1 (residual work item, or the greedy argmax), or n = L
// (bonus draw, or the greedy argmax); residual and bonus draws are made by
// residual_select.  The accept tests are those of the pages in fp64.
// ---------------------------------------------------------------------------
constexpr uint32_t kProgOne = 1u << 20;
constexpr uint32_t kVerifyDone = 0x80000000u;
__device__ __forceinline__ int prog_of(uint32_t w) { return (int)((w >> 20) & 31u); }

// Lane 0 applies the read-modify-write; every lane gets the previous word.
__device__ __forceinline__ uint32_t vstate_or(uint32_t* w, uint32_t bits, int lane) {
  uint32_t old = 0u;
  if (lane == 0) old = __hip_atomic_fetch_or(w, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __shfl(old, 0);
}
__device__ __forceinline__ uint32_t vstate_add(uint32_t* w, uint32_t v, int lane) {
  uint32_t old = 0u;
  if (lane == 0) old = __hip_atomic_fetch_add(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __shfl(old, 0);
}

constexpr int kLazyBlocks = 4;  // 4096-column blocks per work item, one per wavefront

template <typename TL, bool VEC>
__global__ __launch_bounds__(256) void verify_lazy_kernel(VerifyArgs a) {
  __shared__ uint32_t s_word;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B, gamma = a.gamma, V = a.V, nb = a.n_blk;
  const int nch = (nb + kLazyBlocks - 1) / kLazyBlocks;
  const int item = blockIdx.x;
  const int j = item / (B * nch), rest = item - j * (B * nch), b = rest / nch, ch = rest - b * nch;
  const int L = budget_of(a, b);
  if (j > L) return;  // uniform across the workgroup
  if (j == 0 && ch == 0 && tid == 0 && a.budget && (a.budget[b] < 0 || a.budget[b] > gamma))
    flag_status(a.status, kBadBudget);
  uint32_t* const vw = a.vstate + b;
  // Rows 0 and 1 are read without asking: row 0 is always needed and row 1
  // whenever position 1 is accepted, the common case, while the question costs
  // a memory round trip before the item's loads can go out.
  if (j > 1) {
    if (tid == 0) s_word = __hip_atomic_load(vw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_word & kVerifyDone) return;  // decided at an earlier position: row j is not needed
  }

  const int row0 = b * (gamma + 1);
  const TL* trow0 = static_cast<const TL*>(a.target) + (size_t)row0 * V;
  const int32_t* xs = a.draft + (size_t)b * gamma;
  // inputs of the test of position j + 1, which the row's last item runs: the
  // drafted token, its draft log-probability and its target logit, requested
  // now so that they have landed by then
  int x_pre = 0;
  float lq_pre = 0.0f;
  if (wave == 0 && j < L) x_pre = xs[j], lq_pre = a.draft_logq[(size_t)b * gamma + j];
  const int blk = ch * kLazyBlocks + wave;
  if (blk < nb) {
    const BlockStat st = block_stats<TL, VEC>(a, row0 + j, blk, effective_temp(a.temperature[b]), lane);
    if (lane == 0) {
      store_bstat_coherent(a.bstat + (size_t)(row0 + j) * nb + blk, st);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // complete at the agent's coherence point
    }
  }
  float z_pre = 0.0f;
  if (wave == 0 && j < L) z_pre = load_logit(trow0 + (size_t)j * V + min(max(x_pre, 0), V - 1));
  // count the item once every statistic of it is stored, so the item that finds
  // the row's count full reads them all with its coherent loads
  __syncthreads();
  if (wave != 0) return;
  uint32_t before = 0u;
  // names the publication point in the assembly (a comment: no instruction)
  asm volatile(";; dspark publish: row counter" ::: "memory");
  if (lane == 0) before = __hip_atomic_fetch_add(a.rowcnt + row0 + j, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__shfl(before, 0) != (uint32_t)(nch - 1)) return;
  // row j is complete: announce it, and test position j + 1 if its turn has come
  {
    const uint32_t old = vstate_or(vw, 1u << j, lane);
    if ((old & kVerifyDone) || prog_of(old) != j) return;
  }

  const float Tf = checked_temp(a.temperature[b], a.status);
  const bool greedy = !(Tf > 0.0f);
  const double invT = greedy ? 0.0 : 1.0 / (double)Tf;
  const uint32_t off = a.pos_offset ? (uint32_t)a.pos_offset[b] : 0u;
  int n = j;  // rows 0..n complete, positions 1..n accepted
  RowInfo ri;
  for (;;) {
    ri = row_info(a.bstat + (size_t)(row0 + n) * nb, nb, greedy, invT, lane);
    if (n == L) break;  // every drafted position accepted
    const int k = n + 1;
    const bool pre = n == j;  // this item's own row: its prefetched inputs
    const int x = checked_token(pre ? __shfl(x_pre, 0) : xs[n], V, a.status, kBadDraft);
    bool fail;
    if (greedy) {
      fail = x != ri.arg;
    } else {
      const float z = pre ? __shfl(z_pre, 0) : load_logit(trow0 + (size_t)n * V + x);
      const double lp = ((double)z - ri.M) * invT - ri.logS;
      const double lq = pre ? (double)__shfl(lq_pre, 0) : (double)a.draft_logq[(size_t)b * gamma + n];
      const double lnu = log(uniform_from_word(rng_word(a.seed, kAccept, b, k + off, 0)));
      fail = !(lnu < lp - lq);  // accept iff u < min(1, p/q), since ln u < 0
      if (a.debug_logp_logq && lane == 0) {
        a.debug_logp_logq[((size_t)b * gamma + n) * 2] = (float)lp;
        a.debug_logp_logq[((size_t)b * gamma + n) * 2 + 1] = (float)lq;
      }
    }
    if (fail) break;
    const uint32_t old = vstate_add(vw, kProgOne, lane);  // m: n -> k
    if (!(old & (1u << k))) return;  // row k not complete yet: its last item tests position k + 1
    n = k;
  }
  // the final token, n accepted: the greedy argmax here; a bonus or residual
  // draw in residual_select (after the residual pass)
  if (lane == 0) {
    ReqState rs;
    rs.row_max = ri.M, rs.row_logsum = ri.logS, rs.res_mass = 0.0, rs.n = n;
    rs.pending = greedy ? 0 : (n < L ? kDrawResidual : kDrawBonus);
    a.req[b] = rs;
    if (rs.pending == kDrawResidual) a.slot_req[atomicAdd(a.slot_count, 1u)] = b;
  }
  for (int i = lane; i <= gamma; i += 64) {
    int t = -1;
    if (i < n) t = xs[i];
    else if (i == n && greedy) t = ri.arg;
    a.out_tokens[(size_t)b * (gamma + 1) + i] = t;
  }
  if (lane == 0) {
    a.num_accepted[b] = n;
    a.num_emitted[b] = n + 1;
  }
  vstate_or(vw, kVerifyDone, lane);
}

template <typename TF>
__device__ __forceinline__ double dot_range(const TF* h, const TF* w, int k0, int k1) {
  if constexpr (sizeof(TF) == 2) {
    if ((((k1 - k0) | k0) & 7) == 0 && k1 - k0 <= 64) {
      // every load first (one memory round trip); a product of two bf16 values
      // is exact in fp32, and the sum runs in fp64 over four independent chains
      uint4 hv[8], wv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + 8 * i < k1) {
          hv[i] = *reinterpret_cast<const uint4*>(h + k0 + 8 * i);
          wv[i] = *reinterpret_cast<const uint4*>(w + k0 + 8 * i);
        }
      double c[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + 8 * i < k1) {
          const uint32_t hh[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w}, ww[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            c[q] += (double)(__uint_as_float(hh[q] << 16) * __uint_as_float(ww[q] << 16));
            c[q] += (double)(__uint_as_float(hh[q] & 0xffff0000u) * __uint_as_float(ww[q] & 0xffff0000u));
          }
        }
      return (c[0] + c[1]) + (c[2] + c[3]);
    }
  }
  double acc = 0.0;
  for (int k = k0; k < k1; ++k) acc += (double)load_logit(h + k) * (double)load_logit(w + k);
  return acc;
}

// fp64 residual r(v) = max(0, p(v) - q(v)) at one column of the rejected row,
// given the Markov bias of that column.
// xb, zt: the column's backbone and target logits.
__device__ __forceinline__ double residual_from(double xb, double zt, const ReqState& st, double invT, double lse_q,
                                                double bias, double* p_out) {
  const double d = xb + bias;
  const double p = exp((zt - st.row_max) * invT - st.row_logsum);
  const double q = exp(d * invT - lse_q);
  if (p_out) *p_out = p;
  return p > q ? p - q : 0.0;
}

template <typename TL>
__device__ __forceinline__ double residual_at(const VerifyArgs& a, int b, const ReqState& st, double invT,
                                              double lse_q, int v, double bias, double* p_out) {
  const int V = a.V, n = st.n;
  const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (a.gamma + 1) + n) * V;
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * a.gamma + n) * V;
  return residual_from((double)load_logit(brow + v), (double)load_logit(trow + v), st, invT, lse_q, bias, p_out);
}

// One workgroup of 4 wavefronts per request that rejected: block and tile from
// the residual tile masses, column from an fp64 recompute of the chosen tile
// (TileDot for bf16 factors at r = 128 or 256, else the rank split over the
// wavefronts).  Memory round trips on the critical path:
//   1. the request's state with the tile masses of the first 64 blocks (wave w,
//      lane l: tile l of blocks w, w + 4, ...), the masses being independent of
//      the state; the Gumbel values of the three levels are computed while the
//      previous token, the draft log-sum-exp and the masses land;
//   2. the chosen block's tile masses again (an L2 hit);
//   3. the tile's factor rows and U[prev] with its backbone and target logits.
// Block masses sum in the order of the per-block loop (wave by wave, blocks in
// increasing order), and each wave takes one logarithm per lane for its blocks.
template <typename TL, typename TF>
__global__ __launch_bounds__(256) void residual_select_kernel(VerifyArgs a) {
  constexpr int kPer = 16;  // blocks per wavefront in one pass: 64 blocks a pass
  __shared__ double s_val[4], s_tot[4], s_part[4][64], s_gmid[64], s_gleaf[64];
  __shared__ int s_idx[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gamma = a.gamma, V = a.V, nt = a.n_tiles, r = a.r;
  const int nblk = (nt + kTilesPerBlock - 1) / kTilesPerBlock;
  const float* R = a.rsum + (size_t)b * nt;
  const ReqState st = a.req[b];
  float rm[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) rm[i] = R[min((wave + 4 * i) * kTilesPerBlock + lane, nt - 1)];
  // the lazy pass's counters of this request (and the residual work list) go
  // back to zero for the next call: every kernel that used them has finished
  if (tid <= a.gamma) a.rowcnt[(size_t)b * (a.gamma + 1) + tid] = 0u;
  if (tid == 0) a.vstate[b] = 0u;
  if (b == 0 && tid == 0) *a.slot_count = 0u;
  if (!st.pending) return;  // uniform across the workgroup
  const int n = st.n;
  const double invT = 1.0 / (double)a.temperature[b];
  const uint32_t off = a.pos_offset ? (uint32_t)a.pos_offset[b] : 0u;
  const uint32_t rpos = n + 1 + off;
  if (st.pending == kDrawBonus) {  // every drafted position accepted: the bonus from target row n = L
    if (wave == 0) {
      const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (gamma + 1) + n) * V;
      const int y = sample_row(trow, a.bstat + ((size_t)b * (gamma + 1) + n) * a.n_blk, a.n_blk, V, invT, a.seed,
                               b, rpos, lane);
      if (lane == 0) a.out_tokens[(size_t)b * (gamma + 1) + n] = y;
    }
    return;
  }
  const int prev_raw = n == 0 ? a.prev0[b] : a.draft[(size_t)b * gamma + n - 1];
  const double lse_q = a.draft_lse[(size_t)b * gamma + n];
  if (wave == 1) s_gmid[lane] = gumbel(a.seed, kFinalMid, b, rpos, lane);
  if (wave == 2) s_gleaf[lane] = gumbel(a.seed, kFinalLeaf, b, rpos, lane);

  // block masses and the block draw
  double tot = 0.0, best = -INFINITY;
  int bi = 0x7fffffff;
  for (int c0 = 0; c0 < nblk; c0 += 4 * kPer) {
    if (c0 > 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) rm[i] = R[min((c0 + wave + 4 * i) * kTilesPerBlock + lane, nt - 1)];
    }
    const int my_blk = c0 + wave + 4 * lane;  // lane i < kPer: the wave's i-th block of the pass
    const double g = lane < kPer && my_blk < nblk ? gumbel(a.seed, kFinalTop, b, rpos, my_blk) : 0.0;
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int blk = c0 + wave + 4 * i;
      if (blk < nblk) {  // uniform across the wavefront
        const int t = blk * kTilesPerBlock + lane;
        const double rb = wave_sum(t < nt ? (double)rm[i] : 0.0);
        tot += rb;
        if (lane == i) mine = rb;
      }
    }
    double val = -INFINITY;
    int idx = 0x7fffffff;
    if (lane < kPer && my_blk < nblk && mine > 0.0) val = log(mine) + g, idx = my_blk;
    wave_argmax(val, idx);
    if (val > best) best = val, bi = idx;  // passes in increasing block order: ties keep the lowest
  }
  if (lane == 0) s_val[wave] = best, s_idx[wave] = bi, s_tot[wave] = tot;
  __syncthreads();
  tot = (s_tot[0] + s_tot[1]) + (s_tot[2] + s_tot[3]);
  best = -INFINITY, bi = 0x7fffffff;
  for (int w = 0; w < 4; ++w)
    if (s_val[w] > best || (s_val[w] == best && s_idx[w] < bi)) best = s_val[w], bi = s_idx[w];

  const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (gamma + 1) + n) * V;
  if (!(tot > 0.0)) {  // no residual mass: draw from p itself
    if (wave == 0) {
      const int y = sample_row(trow, a.bstat + ((size_t)b * (gamma + 1) + n) * a.n_blk, a.n_blk, V, invT, a.seed,
                               b, rpos, lane);
      if (lane == 0) {
        a.out_tokens[(size_t)b * (gamma + 1) + n] = y;
        a.req[b].res_mass = tot;
      }
    }
    return;
  }
  // tile inside the chosen block (every wavefront, so that none waits for another)
  bi = index_or(bi, nblk, 0);
  const int t0 = bi * kTilesPerBlock, t1 = min(t0 + kTilesPerBlock, nt);
  double val = -INFINITY;
  int ti = 0x7fffffff;
  if (t0 + lane < t1) {
    const float rt = R[t0 + lane];
    if (rt > 0.0f) val = log((double)rt) + s_gmid[lane], ti = t0 + lane;
  }
  wave_argmax(val, ti);
  ti = index_or(ti, t1, t0);

  // Markov bias of the chosen tile in fp64; the column's backbone and target
  // logits come in the same round trip (with bf16 factors at r = 128 or 256,
  // so do the U[prev] chunks)
  const int prev = checked_token(prev_raw, V, a.status, n == 0 ? kBadPrev : kBadDraft);
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  TileDot td;
  td.nj = sizeof(TF) == 2 && (r == 128 || r == 256) ? r / 64 : 0;
  if (td.nj) td.load_h(reinterpret_cast<const uint16_t*>(h), lane);
  const int v = ti * kTile + lane;
  double xb = 0.0, zt = 0.0;
  if (wave == 0 && v < V) {
    const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * gamma + n) * V;
    xb = (double)load_logit(brow + v), zt = (double)load_logit(trow + v);
  }
  if (td.nj) {
    double dt[2];
    td.dot(static_cast<const uint16_t*>(a.Wt), ti * kTile, V, wave, lane, dt);
    if ((lane & 7) == 0) s_part[0][16 * wave + (lane >> 3)] = dt[0], s_part[0][16 * wave + (lane >> 3) + 8] = dt[1];
  } else {
    // the rank split over the four wavefronts
    const int kq = (r + 3) / 4, k0 = min(wave * kq, r), k1 = min(k0 + kq, r);
    s_part[wave][lane] = v < V ? dot_range<TF>(h, static_cast<const TF*>(a.Wt) + (size_t)v * r, k0, k1) : 0.0;
  }
  __syncthreads();
  if (wave != 0) return;
  double lv = -INFINITY, lp = -INFINITY;
  int vi = 0x7fffffff;
  if (v < V) {
    double p;
    const double bias =
        td.nj ? s_part[0][lane] : (s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]);
    const double rv = residual_from(xb, zt, st, invT, lse_q, bias, &p);
    const double g = s_gleaf[lane];
    if (rv > 0.0) lv = log(rv) + g, vi = v;
    lp = log(p) + g;
  }
  wave_argmax(lv, vi);
  if (vi == 0x7fffffff) {  // the chosen tile lost all residual mass in fp64
    vi = v < V ? v : 0x7fffffff;
    wave_argmax(lp, vi);
  }
  const int y = index_or(vi, min(V, (ti + 1) * kTile), ti * kTile);
  if (lane == 0) {
    a.out_tokens[(size_t)b * (gamma + 1) + n] = y;
    a.req[b].res_mass = tot;
  }
}

template <typename TL, typename TF>
__global__ __launch_bounds__(64) void residual_debug_kernel(VerifyArgs a) {
  const int tile = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const ReqState st = a.req[b];
  if (st.pending != kDrawResidual) return;
  const int v = tile * kTile + lane;
  if (v >= a.V) return;
  const int gamma = a.gamma, n = st.n, r = a.r;
  int prev = n == 0 ? a.prev0[b] : a.draft[(size_t)b * gamma + n - 1];
  prev = prev < 0 ? 0 : (prev >= a.V ? a.V - 1 : prev);
  const double invT = 1.0 / (double)a.temperature[b];
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  const double bias = dot_range<TF>(h, static_cast<const TF*>(a.Wt) + (size_t)v * r, 0, r);
  double p;
  const double rv = residual_at<TL>(a, b, st, invT, a.draft_lse[(size_t)b * gamma + n], v, bias, &p);
  a.debug_residual[(size_t)b * a.V + v] = (float)(st.res_mass > 0.0 ? rv / st.res_mass : p);
}

// ---------------------------------------------------------------------------
// Analytic acceptance c*_k = sum_v min(p_k(v), q_k(v)) = 1 - TV(p_k, q_k) at
// every block position ("DSpark, la bozza ...", section "Verificare meglio, non
// di più", eq. c*_k): the tile masses come from the residual-mode GEMM pass in
// its acceptance form; these two kernels prepare the target row statistics and
// add the tile masses up (one wavefront per (request, row)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void row_info_kernel(AcceptanceArgs a) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (s >= a.B * a.gamma) return;  // uniform across the wavefront
  const int b = s / a.gamma, j = s - b * a.gamma;
  const float Tf = checked_temp(a.temperature[b], a.status);
  const bool greedy = !(Tf > 0.0f);
  const RowInfo ri = row_info(a.bstat + ((size_t)b * (a.gamma + 1) + j) * a.n_blk, a.n_blk, greedy,
                              greedy ? 0.0 : 1.0 / (double)Tf, lane);
  if (lane == 0) {
    a.rowinfo[s] = make_double2(ri.M, ri.logS);
    a.rowarg[s] = ri.arg;
  }
}

__global__ __launch_bounds__(256) void acceptance_finish_kernel(AcceptanceArgs a) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (s >= a.B * a.gamma) return;  // uniform across the wavefront
  const int b = s / a.gamma;
  if (!(effective_temp(a.temperature[b]) > 0.0f)) {
    // greedy: both distributions are one-hot at their lowest-index maximum
    if (lane == 0) a.c_star[s] = a.draft[s] == a.rowarg[s] ? 1.0 : 0.0;
    return;
  }
  const float* m = a.tile_mass + (size_t)s * a.n_tiles;  // rows of n_tiles, the first n_parts used
  double acc = 0.0;
  for (int t = lane; t < a.n_parts; t += 64) acc += (double)m[t];
  acc = wave_sum(acc);
  if (lane == 0) a.c_star[s] = acc;
}

}  // namespace

hipError_t launch_row_stats(const VerifyArgs& a, int logits_dtype, hipStream_t s) {
  const dim3 grid(a.n_blk, a.B * (a.gamma + 1));
  if (logits_dtype == DSPARK_BF16) {
    if (a.V % 8 == 0) launch(&row_stats_kernel<uint16_t, true>, grid, 64, 0, s, a);
    else launch(&row_stats_kernel<uint16_t, false>, grid, 64, 0, s, a);
  } else {
    if (a.V % 4 == 0) launch(&row_stats_kernel<float, true>, grid, 64, 0, s, a);
    else launch(&row_stats_kernel<float, false>, grid, 64, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_verify_lazy(const VerifyArgs& a, int logits_dtype, hipStream_t s) {
  const long long items = (long long)(a.gamma + 1) * a.B * ((a.n_blk + kLazyBlocks - 1) / kLazyBlocks);
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)items;
  if (logits_dtype == DSPARK_BF16) {
    if (a.V % 8 == 0) launch(&verify_lazy_kernel<uint16_t, true>, grid, 256, 0, s, a);
    else launch(&verify_lazy_kernel<uint16_t, false>, grid, 256, 0, s, a);
  } else {
    if (a.V % 4 == 0) launch(&verify_lazy_kernel<float, true>, grid, 256, 0, s, a);
    else launch(&verify_lazy_kernel<float, false>, grid, 256, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_residual_select(const VerifyArgs& a, int logits_dtype, int factor_dtype,
                                  hipStream_t s) {
  if (logits_dtype == DSPARK_BF16) {
    if (factor_dtype == DSPARK_BF16) launch(&residual_select_kernel<uint16_t, uint16_t>, a.B, 256, 0, s, a);
    else launch(&residual_select_kernel<uint16_t, float>, a.B, 256, 0, s, a);
  } else {
    if (factor_dtype == DSPARK_BF16) launch(&residual_select_kernel<float, uint16_t>, a.B, 256, 0, s, a);
    else launch(&residual_select_kernel<float, float>, a.B, 256, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_residual_debug(const VerifyArgs& a, int logits_dtype, int factor_dtype,
                                 hipStream_t s) {
  const dim3 grid(a.n_tiles, a.B);
  if (logits_dtype == DSPARK_BF16) {
    if (factor_dtype == DSPARK_BF16) launch(&residual_debug_kernel<uint16_t, uint16_t>, grid, 64, 0, s, a);
    else launch(&residual_debug_kernel<uint16_t, float>, grid, 64, 0, s, a);
  } else {
    if (factor_dtype == DSPARK_BF16) launch(&residual_debug_kernel<float, uint16_t>, grid, 64, 0, s, a);
    else launch(&residual_debug_kernel<float, float>, grid, 64, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_row_info(const AcceptanceArgs& a, hipStream_t s) {
  launch(&row_info_kernel, (a.B * a.gamma + 3) / 4, 256, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_acceptance_finish(const AcceptanceArgs& a, hipStream_t s) {
  launch(&acceptance_finish_kernel, (a.B * a.gamma + 3) / 4, 256, 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark

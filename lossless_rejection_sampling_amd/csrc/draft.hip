// Draft half of the round: the Markov-head bias contraction fused with the
// softmax statistics of every 64-column tile, and the per-request draw of one
// block position.
//
// The draft distribution at block position k is softmax((U_k + B(x_{k-1}, .)) / T)
// with the Markov bias B(x, v) = sum_rho W1[x, rho] W2[rho, v] of rank r
// ("DSpark, la bozza che sa quando fermarsi", section "Un po' di
// autoregressione basta", eq. p_k and the factorisation B = W1 W2).  Here U is
// W1 [V, r] and Wt is W2 stored vocabulary-major [V, r], so both operands of the
// contraction are contiguous along r.
#include <math.h>

#include "dspark.h"
#include "kernels.hpp"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Which request, base row and previous token a GEMM slot stands for.
template <bool RESIDUAL>
__device__ __forceinline__ void slot_info(const GemmArgs& a, int s, int nslots, int& b, int& pos,
                                          int& prev, bool& valid) {
  valid = s < nslots;
  if (RESIDUAL) {
    b = valid ? a.slot_req[s] : 0;
    pos = valid ? a.req[b].n : 0;
  } else {
    b = valid ? s : 0;
    pos = a.pos;
  }
  int pv = pos == 0 ? a.prev0[b] : a.draft[(size_t)b * a.gamma + pos - 1];
  prev = valid ? checked_token(pv, a.V, a.status, pos == 0 ? kBadPrev : kBadDraft) : 0;
}

// Four consecutive logits [v, v+4) of one row; missing columns read as -inf.
template <typename TL, bool VEC>
__device__ __forceinline__ void load4(const TL* row, int v, int V, float out[4]) {
  if (VEC && v + 4 <= V) {
    if constexpr (sizeof(TL) == 2) {
      const u16x4 h = *reinterpret_cast<const u16x4*>(row + v);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = bf16_bits_to_f32(h[e]);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(row + v);
      out[0] = f.x, out[1] = f.y, out[2] = f.z, out[3] = f.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (v + e < V) ? load_logit(row + v + e) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// MFMA path (bf16 factors, r a multiple of 16).
//
// A workgroup of 4 wavefronts owns one 64-column tile and 256 slots; each
// wavefront computes the [64 columns x 64 slots] bias block as 2 x 2
// v_mfma_f32_32x32x16_bf16 tiles with A = Wt rows (columns v) and B = gathered
// U rows (slots).  In the accumulator layout a lane holds, for slot (lane % 32),
// 16 of the 32 columns of each 32-column block, so the per-(slot, tile)
// statistics reduce within the lane and then with its partner lane (lane ^ 32).
// ---------------------------------------------------------------------------
template <typename TL, bool RESIDUAL, bool VEC>
__global__ __launch_bounds__(256) void gemm_stats_mfma(GemmArgs a) {
  const int tile = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int slot0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * 64;
  const int nslots = RESIDUAL ? (int)*a.slot_count : a.B;
  if (slot0 >= nslots) return;  // uniform across the wavefront
  const int half = lane >> 5, l32 = lane & 31;
  const int V = a.V, r = a.r;
  const int v0 = tile * kTile;

  int b[2], pos[2], prev[2];
  bool valid[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) slot_info<RESIDUAL>(a, slot0 + bb * 32 + l32, nslots, b[bb], pos[bb], prev[bb], valid[bb]);

  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);
  const uint16_t* U = static_cast<const uint16_t*>(a.U);
  const uint16_t* arow[2];
  bool aok[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    const int v = v0 + vb * 32 + l32;
    aok[vb] = v < V;
    arow[vb] = Wt + (size_t)(aok[vb] ? v : 0) * r + half * 8;
  }
  const uint16_t* brow[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) brow[bb] = U + (size_t)prev[bb] * r + half * 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const bf16x8 zero = {};
  for (int k = 0; k < r; k += 16) {
    bf16x8 A[2], Bv[2];
#pragma unroll
    for (int vb = 0; vb < 2; ++vb) A[vb] = aok[vb] ? *reinterpret_cast<const bf16x8*>(arow[vb] + k) : zero;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) Bv[bb] = valid[bb] ? *reinterpret_cast<const bf16x8*>(brow[bb] + k) : zero;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
        acc[vb][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[vb], Bv[bb], acc[vb][bb], 0, 0, 0);
  }

  // Epilogue.  Accumulator element e of block (vb, bb) is column
  // v0 + vb*32 + 8*(e/4) + 4*half + e%4 of slot bb*32 + l32.
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int rq = b[bb];
    const float T = valid[bb] ? effective_temp(a.temperature[rq]) : 1.0f;
    const bool sampled = T > 0.0f;
    const TL* brow_l = static_cast<const TL*>(a.base) + ((size_t)rq * a.gamma + pos[bb]) * V;
    float x[2][16];
    float ref = -INFINITY;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        load4<TL, VEC>(brow_l, v0 + vb * 32 + g * 8 + half * 4, V, &x[vb][g * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) ref = fmaxf(ref, x[vb][g * 4 + e]);
      }
    ref = fmaxf(ref, __shfl_xor(ref, 32));
    float tmax = -INFINITY;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[vb][e] = (x[vb][e] - ref) + acc[vb][bb][e];  // -inf stays -inf for missing columns
        tmax = fmaxf(tmax, x[vb][e]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if constexpr (!RESIDUAL) {
      const float c = sampled ? kLog2e / T : 0.0f;
      float s = 0.0f;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += exp2f((x[vb][e] - tmax) * c);
      s += __shfl_xor(s, 32);
      if (half == 0 && valid[bb]) {
        TileStat st;
        st.ref = ref, st.mx = tmax, st.sum = s, st.pad = 0.0f;
        a.tstat[(size_t)rq * a.n_tiles + tile] = st;
      }
    } else {
      // r(v) = max(0, p(v) - q(v)) with p from the target row and q rebuilt from
      // the draft statistics of the same position.
      float rs = 0.0f;
      if (valid[bb]) {
        const ReqState st = a.req[rq];
        const float invT = 1.0f / T;
        const float mp = (float)st.row_max, lsp = (float)st.row_logsum;
        const double lse_q = a.draft_lse[(size_t)rq * a.gamma + pos[bb]];
        const float cq = (float)(lse_q - (double)ref / (double)T);
        const TL* trow = static_cast<const TL*>(a.target) + ((size_t)rq * (a.gamma + 1) + pos[bb]) * V;
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float z[4];
            load4<TL, VEC>(trow, v0 + vb * 32 + g * 8 + half * 4, V, z);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = expf((z[e] - mp) * invT - lsp);
              const float q = expf(x[vb][g * 4 + e] * invT - cq);
              rs += fmaxf(p - q, 0.0f);
            }
          }
      }
      rs += __shfl_xor(rs, 32);
      if (half == 0 && valid[bb]) a.rsum[(size_t)rq * a.n_tiles + tile] = rs;
    }
  }
}

// ---------------------------------------------------------------------------
// VALU path (any factor type and rank): one wavefront per (slot, tile), one
// column per lane.
// ---------------------------------------------------------------------------
template <typename TL, typename TF, bool RESIDUAL>
__global__ __launch_bounds__(64) void gemm_stats_valu(GemmArgs a) {
  const int tile = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int nslots = RESIDUAL ? (int)*a.slot_count : a.B;
  if (s >= nslots) return;
  int b, pos, prev;
  bool valid;
  slot_info<RESIDUAL>(a, s, nslots, b, pos, prev, valid);
  const int V = a.V, r = a.r;
  const int v = tile * kTile + lane;
  const bool ok = v < V;
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  const TF* w = static_cast<const TF*>(a.Wt) + (size_t)(ok ? v : 0) * r;
  float bias = 0.0f;
  for (int k = 0; k < r; ++k) bias = fmaf(load_logit(h + k), load_logit(w + k), bias);
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * a.gamma + pos) * V;
  const float x = ok ? load_logit(brow + v) : -INFINITY;
  const float ref = wave_max(x);
  const float t = ok ? (x - ref) + bias : -INFINITY;
  const float tmax = wave_max(t);
  const float T = effective_temp(a.temperature[b]);
  if constexpr (!RESIDUAL) {
    const float c = T > 0.0f ? kLog2e / T : 0.0f;
    const float sum = wave_sum(ok ? exp2f((t - tmax) * c) : 0.0f);
    if (lane == 0) {
      TileStat st;
      st.ref = ref, st.mx = tmax, st.sum = sum, st.pad = 0.0f;
      a.tstat[(size_t)b * a.n_tiles + tile] = st;
    }
  } else {
    const ReqState st = a.req[b];
    const float invT = 1.0f / T;
    const double lse_q = a.draft_lse[(size_t)b * a.gamma + pos];
    const float cq = (float)(lse_q - (double)ref / (double)T);
    float rv = 0.0f;
    if (ok) {
      const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (a.gamma + 1) + pos) * V;
      const float p = expf((load_logit(trow + v) - (float)st.row_max) * invT - (float)st.row_logsum);
      const float q = expf(t * invT - cq);
      rv = fmaxf(p - q, 0.0f);
    }
    const float sum = wave_sum(rv);
    if (lane == 0) a.rsum[(size_t)b * a.n_tiles + tile] = sum;
  }
}

// ---------------------------------------------------------------------------
// One draw per request at block position pos+1: three-level Gumbel-max over
// blocks of 64 tiles, tiles of 64 columns, and columns, from the tile
// statistics; the chosen tile is recomputed in fp64.  Greedy requests take the
// tile with the largest logit and its argmax (lowest index on ties).
// ---------------------------------------------------------------------------
template <typename TL, typename TF>
__global__ __launch_bounds__(64) void draft_select_kernel(DraftSelectArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int V = a.V, r = a.r, gamma = a.gamma, nt = a.n_tiles, pos = a.pos;
  const uint32_t rpos = (uint32_t)(pos + 1 + (a.pos_offset ? a.pos_offset[b] : 0));
  const float Tf = checked_temp(a.temperature[b], a.status);
  int prev = pos == 0 ? a.prev0[b] : a.draft[(size_t)b * gamma + pos - 1];
  prev = checked_token(prev, V, a.status, pos == 0 ? kBadPrev : kBadDraft);
  const TileStat* ts = a.tstat + (size_t)b * nt;
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * gamma + pos) * V;
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  const TF* Wt = static_cast<const TF*>(a.Wt);

  auto recompute = [&](int v) -> double {  // d(v) in fp64
    const TF* w = Wt + (size_t)v * r;
    double acc = 0.0;
    for (int k = 0; k < r; ++k) acc += (double)load_logit(h + k) * (double)load_logit(w + k);
    return (double)load_logit(brow + v) + acc;
  };

  int x;
  double logq, lse;
  if (Tf > 0.0f) {
    const double invT = 1.0 / (double)Tf;
    const double mref = (double)ts[0].ref + (double)ts[0].mx;
    const int nblk = (nt + kTilesPerBlock - 1) / kTilesPerBlock;
    double row_m = -INFINITY, row_s = 0.0, best = -INFINITY;
    int best_blk = 0x7fffffff;
    for (int g = 0; g < nblk; g += 64) {
      const int blk = g + lane;
      if (blk < nblk) {
        const int t0 = blk * kTilesPerBlock, t1 = min(t0 + kTilesPerBlock, nt);
        double dmax = -INFINITY;
        for (int t = t0; t < t1; ++t) dmax = fmax(dmax, (double)ts[t].ref + (double)ts[t].mx);
        float s = 0.0f;
        for (int t = t0; t < t1; ++t)
          s += ts[t].sum * expf((float)(((double)ts[t].ref + (double)ts[t].mx - dmax) * invT));
        const double val = (dmax - mref) * invT + log((double)s) + gumbel(a.seed, kDraftTop, b, rpos, blk);
        if (val > best) best = val, best_blk = blk;
        if (dmax > row_m) {
          row_s = row_s * exp((row_m - dmax) * invT) + s;
          row_m = dmax;
        } else {
          row_s += s * exp((dmax - row_m) * invT);
        }
      }
    }
    wave_argmax(best, best_blk);
    best_blk = index_or(best_blk, nblk, 0);
    const double M = wave_max(row_m);
    const double S = wave_sum(row_s > 0.0 ? row_s * exp((row_m - M) * invT) : 0.0);
    lse = M * invT + log(S);

    const int t0 = best_blk * kTilesPerBlock, t1 = min(t0 + kTilesPerBlock, nt);
    double val = -INFINITY;
    int ti = 0x7fffffff;
    if (t0 + lane < t1) {
      const TileStat st = ts[t0 + lane];
      val = ((double)st.ref + (double)st.mx - mref) * invT + log((double)st.sum) +
            gumbel(a.seed, kDraftMid, b, rpos, lane);
      ti = t0 + lane;
    }
    wave_argmax(val, ti);
    ti = index_or(ti, nt, t0);

    const int v = ti * kTile + lane;
    double sv = -INFINITY, lv = -INFINITY;
    int vi = 0x7fffffff;
    if (v < V) {
      sv = recompute(v) / (double)Tf;
      lv = sv + gumbel(a.seed, kDraftLeaf, b, rpos, lane);
      vi = v;
    }
    wave_argmax(lv, vi);
    x = index_or(vi, min(V, (ti + 1) * kTile), ti * kTile);
    const double sx = __shfl(sv, x - ti * kTile);
    logq = sx - lse;
  } else {
    double best = -INFINITY;
    int bt = 0x7fffffff;
    for (int t = lane; t < nt; t += 64) {
      const double d = (double)ts[t].ref + (double)ts[t].mx;
      if (d > best) best = d, bt = t;
    }
    wave_argmax(best, bt);
    bt = index_or(bt, nt, 0);
    const int v = bt * kTile + lane;
    double d = -INFINITY;
    int vi = 0x7fffffff;
    if (v < V) d = recompute(v), vi = v;
    wave_argmax(d, vi);
    x = index_or(vi, min(V, (bt + 1) * kTile), bt * kTile);
    logq = 0.0;
    lse = d;
  }
  if (lane == 0) {
    a.draft[(size_t)b * gamma + pos] = x;
    a.logq[(size_t)b * gamma + pos] = (float)logq;
    a.lse[(size_t)b * gamma + pos] = lse;
  }
}

template <typename TL, bool RESIDUAL>
hipError_t gemm_dispatch(const GemmArgs& a, int factor_dtype, bool vec, hipStream_t s) {
  if (factor_dtype == DSPARK_BF16 && a.r % 16 == 0) {
    const dim3 grid(a.n_tiles, (a.B + 255) / 256);
    if (vec) gemm_stats_mfma<TL, RESIDUAL, true><<<grid, 256, 0, s>>>(a);
    else gemm_stats_mfma<TL, RESIDUAL, false><<<grid, 256, 0, s>>>(a);
  } else {
    const dim3 grid(a.n_tiles, a.B);
    if (factor_dtype == DSPARK_BF16) gemm_stats_valu<TL, uint16_t, RESIDUAL><<<grid, 64, 0, s>>>(a);
    else gemm_stats_valu<TL, float, RESIDUAL><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_stats(const GemmArgs& a, int logits_dtype, int factor_dtype, bool residual,
                             hipStream_t s) {
  const bool vec = a.V % 4 == 0;
  if (logits_dtype == DSPARK_BF16)
    return residual ? gemm_dispatch<uint16_t, true>(a, factor_dtype, vec, s)
                    : gemm_dispatch<uint16_t, false>(a, factor_dtype, vec, s);
  return residual ? gemm_dispatch<float, true>(a, factor_dtype, vec, s)
                  : gemm_dispatch<float, false>(a, factor_dtype, vec, s);
}

hipError_t launch_draft_select(const DraftSelectArgs& a, int logits_dtype, int factor_dtype,
                               hipStream_t s) {
  const dim3 grid(a.B);
  if (logits_dtype == DSPARK_BF16) {
    if (factor_dtype == DSPARK_BF16) draft_select_kernel<uint16_t, uint16_t><<<grid, 64, 0, s>>>(a);
    else draft_select_kernel<uint16_t, float><<<grid, 64, 0, s>>>(a);
  } else {
    if (factor_dtype == DSPARK_BF16) draft_select_kernel<float, uint16_t><<<grid, 64, 0, s>>>(a);
    else draft_select_kernel<float, float><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dspark

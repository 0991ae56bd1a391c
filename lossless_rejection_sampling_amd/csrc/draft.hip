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

constexpr int kSlotsPerGroup = 256;

// ---------------------------------------------------------------------------
// Pipelined MFMA path (bf16 factors, R in {64, 128, 256}): the main kernel.
//
// Workgroup = 8 wavefronts (two per SIMD), wave w owning slots sg0 + 32w .. +31
// of a 256-slot group (grid.y); grid.x is a persistent index over 64-column
// tiles, all wavefronts of a workgroup working on the same tile.
//   * B operands: the gathered rows h_s = U[prev_s] of the wave's 32 slots stay
//     in registers for the whole kernel.
//   * A operands: the tile's W2 rows are streamed into a two-slot LDS ring by
//     direct global->LDS loads, laid out as operand blocks (column block vb,
//     k-step ks) of 64 lanes x 16 B, so each MFMA operand is one conflict-free
//     1 KB ds_read_b128.
//   * The backbone logits the epilogue needs are loaded one tile ahead into
//     registers (the residual pass loads its target logits at the start of
//     the epilogue).  Only the last tile can be ragged; it takes a
//     separate, masked load path so the loop has no per-lane branches around
//     its loads.
//   * Iteration i issues the W2 load of tile i+2, the logits of tile i+1 and the
//     MFMAs of tile i+1, then runs the softmax epilogue of tile i; the barrier
//     at its end waits only for the W2 load, the oldest outstanding one.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kLdsWaves = 8;

// Logits of one tile for one 32-slot block: 2 column blocks x 16 accumulator
// rows, as loaded (bf16 pairs per 32-bit register, or fp32); missing columns
// read as -inf.
template <typename TL> struct TileBuf;
template <> struct TileBuf<uint16_t> {
  uint32_t w[2][8];
  __device__ __forceinline__ float get(int vb, int e) const {
    const uint32_t u = w[vb][e >> 1];
    return (e & 1) ? __uint_as_float(u & 0xffff0000u) : __uint_as_float(u << 16);
  }
};
template <> struct TileBuf<float> {
  float f[2][16];
  __device__ __forceinline__ float get(int vb, int e) const { return f[vb][e]; }
};

// Loads of one tile: `full` (uniform) selects unmasked vector loads.
template <typename TL>
__device__ __forceinline__ void load_tile(const TL* row, int v0, int half, int V, bool full, TileBuf<TL>& x) {
  if (full) {
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const TL* p = row + v0 + vb * 32 + g * 8 + half * 4;
        if constexpr (sizeof(TL) == 2) {
          const uint2 u = *reinterpret_cast<const uint2*>(p);
          x.w[vb][2 * g] = u.x, x.w[vb][2 * g + 1] = u.y;
        } else {
          const float4 f = *reinterpret_cast<const float4*>(p);
          x.f[vb][4 * g] = f.x, x.f[vb][4 * g + 1] = f.y, x.f[vb][4 * g + 2] = f.z, x.f[vb][4 * g + 3] = f.w;
        }
      }
  } else {
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v = v0 + vb * 32 + g * 8 + half * 4;
        if constexpr (sizeof(TL) == 2) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (v + e < V) ? (uint32_t)row[v + e] : 0xff80u;
          x.w[vb][2 * g] = h[0] | (h[1] << 16), x.w[vb][2 * g + 1] = h[2] | (h[3] << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x.f[vb][4 * g + e] = (v + e < V) ? row[v + e] : -INFINITY;
        }
      }
  }
}

template <typename TL, bool RESIDUAL>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const f32x16 (&acc)[2], const TileBuf<TL>& x,
                                              const TL* trow, int rq, int pos, bool valid, float T, int tile,
                                              int half, bool full) {
  float ref = -INFINITY;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) ref = fmaxf(ref, x.get(vb, e));
  ref = fmaxf(ref, __shfl_xor(ref, 32));
  float t[2][16];
  float tmax = -INFINITY;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      t[vb][e] = (x.get(vb, e) - ref) + acc[vb][e];
      tmax = fmaxf(tmax, t[vb][e]);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  if constexpr (!RESIDUAL) {
    const float c = T > 0.0f ? kLog2e / T : 0.0f;
    const float mc = tmax * c;
    float s = 0.0f;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += __builtin_amdgcn_exp2f(fmaf(t[vb][e], c, -mc));
    s += __shfl_xor(s, 32);
    if (half == 0 && valid) {
      TileStat st;
      st.ref = ref, st.mx = tmax, st.sum = s, st.pad = 0.0f;
      a.tstat[(size_t)rq * a.n_tiles + tile] = st;
    }
  } else {
    TileBuf<TL> z;
    load_tile<TL>(trow, tile * kTile, half, a.V, full, z);
    float rs = 0.0f;
    if (valid) {
      const ReqState st = a.req[rq];
      const float c = kLog2e / T;
      const float kp = (float)(((double)st.row_max / (double)T + st.row_logsum) * 1.4426950408889634);
      const double lse_q = a.draft_lse[(size_t)rq * a.gamma + pos];
      const float kq = (float)((lse_q - (double)ref / (double)T) * 1.4426950408889634);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(z.get(vb, e), c, -kp));
          const float q = __builtin_amdgcn_exp2f(fmaf(t[vb][e], c, -kq));
          rs += fmaxf(p - q, 0.0f);
        }
    }
    rs += __shfl_xor(rs, 32);
    if (half == 0 && valid) a.rsum[(size_t)rq * a.n_tiles + tile] = rs;
  }
}

template <typename TL, bool RESIDUAL, int R>
__global__ __launch_bounds__(512, 1) void gemm_stats_lds(GemmArgs a) {
  constexpr int KS = R / 16, NBLK = 2 * KS, TILE_BYTES = NBLK * 1024;
  constexpr bool PF = true;  // backbone logits prefetched a tile ahead (the residual pass
                             // loads its target logits at the start of the epilogue)
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nslots = RESIDUAL ? (int)*a.slot_count : a.B;
  const int sg0 = blockIdx.y * kSlotsPerGroup;
  const int nt = a.n_tiles, G = gridDim.x;
  if (sg0 >= nslots || (int)blockIdx.x >= nt) return;  // uniform across the workgroup
  const int V = a.V;
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);

  // this wave's 32 slots: request, row, temperature and gathered U row
  const bool active = sg0 + wave * 32 < nslots;
  int rq, pos, prev;
  bool valid;
  slot_info<RESIDUAL>(a, sg0 + wave * 32 + l32, nslots, rq, pos, prev, valid);
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)rq * a.gamma + pos) * V;
  const TL* trow = RESIDUAL ? static_cast<const TL*>(a.target) + ((size_t)rq * (a.gamma + 1) + pos) * V : brow;
  const float T = valid ? effective_temp(a.temperature[rq]) : 1.0f;
  bf16x8 H[KS];
  {
    const uint16_t* h = static_cast<const uint16_t*>(a.U) + (size_t)prev * R + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 zero = {};
      H[ks] = valid ? *reinterpret_cast<const bf16x8*>(h + ks * 16) : zero;
    }
  }

  auto fill = [&](int tile, int buf) {  // this wave's share of the tile's operand blocks
    for (int j = wave; j < NBLK; j += nwaves) {
      const int vb = j / KS, ks = j - vb * KS;
      int v = tile * kTile + vb * 32 + l32;
      v = v < V ? v : V - 1;  // columns beyond V are masked in the epilogue
      __builtin_amdgcn_global_load_lds(Wt + (size_t)v * R + ks * 16 + half * 8,
                                       (lds_ptr_t)(lds + buf * TILE_BYTES + j * 1024), 16, 0, 0);
    }
  };
  auto mma = [&](int buf, f32x16 (&acc)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    const char* base = lds + buf * TILE_BYTES + lane * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 A[2];
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) A[vb] = *reinterpret_cast<const bf16x8*>(base + (vb * KS + ks) * 1024);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[vb], H[ks], acc[vb], 0, 0, 0);
    }
  };
  auto full_tile = [&](int tile) { return (tile + 1) * kTile <= V; };
  // Wait until at most `newer` vector-memory loads issued after the W2 fill are
  // still in flight (loads complete in order), then synchronise the workgroup.
  auto sync_fill = [&](bool wait_all) {
    if (wait_all) __builtin_amdgcn_s_waitcnt(0xF70);        // vmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0xF70 | 8);             // vmcnt(8): the 8 logit loads may stay in flight
    __syncthreads();
  };

  f32x16 acc0[2], acc1[2];
  TileBuf<TL> x0, x1;
  int t = blockIdx.x;
  fill(t, 0);
  if (PF && active) load_tile<TL>(brow, t * kTile, half, V, full_tile(t), x0);
  sync_fill(true);
  if (t + G < nt) fill(t + G, 1);
  if (active) mma(0, acc0);
  sync_fill(true);

  for (;;) {
    // tile t: acc0, x0, W2 buffer 0; tile t+G ready in buffer 1
    if (t + 2 * G < nt) fill(t + 2 * G, 0);
    const bool more = t + G < nt;
    if (more && active) {
      if (PF) load_tile<TL>(brow, (t + G) * kTile, half, V, full_tile(t + G), x1);
      mma(1, acc1);
    }
    if (active) epilogue_tile<TL, RESIDUAL>(a, acc0, x0, trow, rq, pos, valid, T, t, half, full_tile(t));
    sync_fill(!(PF && more && active && full_tile(t + G)));
    t += G;
    if (t >= nt) break;
    // tile t: acc1, x1, buffer 1; tile t+G ready in buffer 0
    if (t + 2 * G < nt) fill(t + 2 * G, 1);
    const bool more2 = t + G < nt;
    if (more2 && active) {
      if (PF) load_tile<TL>(brow, (t + G) * kTile, half, V, full_tile(t + G), x0);
      mma(0, acc0);
    }
    if (active) epilogue_tile<TL, RESIDUAL>(a, acc1, x1, trow, rq, pos, valid, T, t, half, full_tile(t));
    sync_fill(!(PF && more2 && active && full_tile(t + G)));
    t += G;
    if (t >= nt) break;
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
// One draw per request at block position pos+1 (a workgroup of 4 wavefronts
// per request): three-level Gumbel-max over blocks of 64 tiles, tiles of 64
// columns, and columns.  Block and tile levels use the tile statistics (one
// coalesced 1 KB read per block); the chosen tile is recomputed in fp64 with
// the rank split over the four wavefronts.  Greedy requests take the tile with
// the largest logit and its argmax (lowest index on ties).
// ---------------------------------------------------------------------------
template <typename TF>
__device__ __forceinline__ double dot_part(const TF* h, const TF* w, int k0, int k1) {
  double acc = 0.0;
  if constexpr (sizeof(TF) == 2) {
    if (((k1 - k0) & 7) == 0 && (k0 & 7) == 0) {
      for (int k = k0; k < k1; k += 8) {
        const uint4 hv = *reinterpret_cast<const uint4*>(h + k);
        const uint4 wv = *reinterpret_cast<const uint4*>(w + k);
        const uint32_t hh[4] = {hv.x, hv.y, hv.z, hv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc += (double)__uint_as_float(hh[q] << 16) * (double)__uint_as_float(ww[q] << 16);
          acc += (double)__uint_as_float(hh[q] & 0xffff0000u) * (double)__uint_as_float(ww[q] & 0xffff0000u);
        }
      }
      return acc;
    }
  }
  for (int k = k0; k < k1; ++k) acc += (double)load_logit(h + k) * (double)load_logit(w + k);
  return acc;
}

template <typename TL, typename TF>
__global__ __launch_bounds__(256) void draft_select_kernel(DraftSelectArgs a) {
  __shared__ double s_val[4], s_m[4], s_s[4], s_part[4][64];
  __shared__ int s_idx[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, r = a.r, gamma = a.gamma, nt = a.n_tiles, pos = a.pos;
  const uint32_t rpos = (uint32_t)(pos + 1 + (a.pos_offset ? a.pos_offset[b] : 0));
  const float Tf = checked_temp(a.temperature[b], a.status);
  int prev = pos == 0 ? a.prev0[b] : a.draft[(size_t)b * gamma + pos - 1];
  prev = checked_token(prev, V, a.status, pos == 0 ? kBadPrev : kBadDraft);
  const TileStat* ts = a.tstat + (size_t)b * nt;
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * gamma + pos) * V;
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  const TF* Wt = static_cast<const TF*>(a.Wt);
  const int nblk = (nt + kTilesPerBlock - 1) / kTilesPerBlock;

  int tile;  // chosen tile
  double invT = 0.0, lse = 0.0;
  if (Tf > 0.0f) {
    invT = 1.0 / (double)Tf;
    const double mref = (double)ts[0].ref + (double)ts[0].mx;
    double best = -INFINITY, row_m = -INFINITY, row_s = 0.0;
    int best_blk = 0x7fffffff;
    for (int blk = wave; blk < nblk; blk += 4) {
      const int t = blk * kTilesPerBlock + lane;
      double d = -INFINITY;
      float sum = 0.0f;
      if (t < nt) {
        const TileStat st = ts[t];
        d = (double)st.ref + (double)st.mx;
        sum = st.sum;
      }
      const double dmax = wave_max(d);
      const float e = t < nt ? sum * expf((float)((d - dmax) * invT)) : 0.0f;
      const double sblk = (double)wave_sum(e);
      const double val = (dmax - mref) * invT + log(sblk) + gumbel(a.seed, kDraftTop, b, rpos, blk);
      if (val > best) best = val, best_blk = blk;
      if (dmax > row_m) {
        row_s = row_s * exp((row_m - dmax) * invT) + sblk;
        row_m = dmax;
      } else {
        row_s += sblk * exp((dmax - row_m) * invT);
      }
    }
    if (lane == 0) s_val[wave] = best, s_idx[wave] = best_blk, s_m[wave] = row_m, s_s[wave] = row_s;
    __syncthreads();
    double M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmax(M, s_m[w]);
    double S = 0.0;
    for (int w = 0; w < 4; ++w)
      if (s_s[w] > 0.0) S += s_s[w] * exp((s_m[w] - M) * invT);
    lse = M * invT + log(S);
    best = -INFINITY, best_blk = 0x7fffffff;
    for (int w = 0; w < 4; ++w)
      if (s_val[w] > best || (s_val[w] == best && s_idx[w] < best_blk)) best = s_val[w], best_blk = s_idx[w];
    best_blk = index_or(best_blk, nblk, 0);
    // tile inside the chosen block (every wavefront computes the same choice)
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
    tile = index_or(ti, t1, t0);
  } else {
    double best = -INFINITY;
    int bt = 0x7fffffff;
    for (int t = tid; t < nt; t += 256) {
      const double d = (double)ts[t].ref + (double)ts[t].mx;
      if (d > best) best = d, bt = t;
    }
    wave_argmax(best, bt);
    if (lane == 0) s_val[wave] = best, s_idx[wave] = bt;
    __syncthreads();
    best = -INFINITY, bt = 0x7fffffff;
    for (int w = 0; w < 4; ++w)
      if (s_val[w] > best || (s_val[w] == best && s_idx[w] < bt)) best = s_val[w], bt = s_idx[w];
    tile = index_or(bt, nt, 0);
  }

  // recompute the chosen tile in fp64: the rank is split over the wavefronts
  const int v = tile * kTile + lane;
  const int kq = (r + 3) / 4, k0 = min(wave * kq, r), k1 = min(k0 + kq, r);
  s_part[wave][lane] = v < V ? dot_part<TF>(h, Wt + (size_t)v * r, k0, k1) : 0.0;
  __syncthreads();
  if (wave == 0) {
    double lv = -INFINITY, sv = -INFINITY;
    int vi = 0x7fffffff;
    if (v < V) {
      const double d = (double)load_logit(brow + v) + ((s_part[0][lane] + s_part[1][lane]) +
                                                       (s_part[2][lane] + s_part[3][lane]));
      if (Tf > 0.0f) {
        sv = d / (double)Tf;
        lv = sv + gumbel(a.seed, kDraftLeaf, b, rpos, lane);
      } else {
        sv = d;
        lv = d;
      }
      vi = v;
    }
    wave_argmax(lv, vi);
    const int x = index_or(vi, min(V, (tile + 1) * kTile), tile * kTile);
    const double sx = __shfl(sv, x - tile * kTile);
    if (lane == 0) {
      a.draft[(size_t)b * gamma + pos] = x;
      a.logq[(size_t)b * gamma + pos] = Tf > 0.0f ? (float)(sx - lse) : 0.0f;
      a.lse[(size_t)b * gamma + pos] = Tf > 0.0f ? lse : sx;
    }
  }
}

template <typename TL, bool RESIDUAL, int R>
hipError_t launch_pipelined(const GemmArgs& a, hipStream_t s) {
  static int max_wg = 0;
  const size_t lds = (size_t)2 * (2 * (R / 16) * 1024);
  const void* fn = reinterpret_cast<const void*>(&gemm_stats_lds<TL, RESIDUAL, R>);
  if (!max_wg) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorUnknown;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * kLdsWaves, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    max_wg = cus * per_cu;
  }
  const int groups = (a.B + kSlotsPerGroup - 1) / kSlotsPerGroup;
  const int threads = 64 * min(kLdsWaves, (a.B + 31) / 32);
  const int wg_x = max(1, min(a.n_tiles, max_wg / groups));
  gemm_stats_lds<TL, RESIDUAL, R><<<dim3(wg_x, groups), threads, lds, s>>>(a);
  return hipGetLastError();
}

template <typename TL, bool RESIDUAL>
hipError_t gemm_dispatch(const GemmArgs& a, int factor_dtype, bool vec, hipStream_t s) {
  if (factor_dtype == DSPARK_BF16 && vec && (a.r == 64 || a.r == 128 || a.r == 256)) {
    if (a.r == 256) return launch_pipelined<TL, RESIDUAL, 256>(a, s);
    if (a.r == 128) return launch_pipelined<TL, RESIDUAL, 128>(a, s);
    return launch_pipelined<TL, RESIDUAL, 64>(a, s);
  }
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
    if (factor_dtype == DSPARK_BF16) draft_select_kernel<uint16_t, uint16_t><<<grid, 256, 0, s>>>(a);
    else draft_select_kernel<uint16_t, float><<<grid, 256, 0, s>>>(a);
  } else {
    if (factor_dtype == DSPARK_BF16) draft_select_kernel<float, uint16_t><<<grid, 256, 0, s>>>(a);
    else draft_select_kernel<float, float><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dspark

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

#include <type_traits>

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

// Loads of one tile, branch-free: every lane issues its 8 vector loads, with
// column addresses clamped into the row (V is a multiple of 4 on this path);
// columns at or beyond V are masked by the epilogue of the (single) ragged tile.
template <typename TL>
__device__ __forceinline__ void load_tile(const TL* row, int v0, int half, int V, TileBuf<TL>& x) {
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int v = min(v0 + vb * 32 + g * 8 + half * 4, V - 4);
      const TL* p = row + v;
      if constexpr (sizeof(TL) == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        x.w[vb][2 * g] = u.x, x.w[vb][2 * g + 1] = u.y;
      } else {
        const float4 f = *reinterpret_cast<const float4*>(p);
        x.f[vb][4 * g] = f.x, x.f[vb][4 * g + 1] = f.y, x.f[vb][4 * g + 2] = f.z, x.f[vb][4 * g + 3] = f.w;
      }
    }
}

// Column of accumulator element e of column block vb (see the MFMA layout).
__device__ __forceinline__ int acc_col(int v0, int vb, int e, int half) {
  return v0 + vb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
}

template <typename TL, bool RESIDUAL>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& a, const f32x16 (&acc)[2], const TileBuf<TL>& x,
                                              const TL* trow, int rq, int pos, bool valid, float T, int tile,
                                              int half, bool full) {
  float xv[2][16];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) xv[vb][e] = x.get(vb, e);
  if (!full) {  // the ragged last tile: columns >= V do not exist
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (acc_col(tile * kTile, vb, e, half) >= a.V) xv[vb][e] = -INFINITY;
  }
  float ref = -INFINITY;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) ref = fmaxf(ref, xv[vb][e]);
  ref = fmaxf(ref, __shfl_xor(ref, 32));
  float t[2][16];
  float tmax = -INFINITY;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      t[vb][e] = (xv[vb][e] - ref) + acc[vb][e];
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
    load_tile<TL>(trow, tile * kTile, half, a.V, z);
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
          const float zv = (full || acc_col(tile * kTile, vb, e, half) < a.V) ? z.get(vb, e) : -INFINITY;
          const float p = __builtin_amdgcn_exp2f(fmaf(zv, c, -kp));
          const float q = __builtin_amdgcn_exp2f(fmaf(t[vb][e], c, -kq));
          rs += fmaxf(p - q, 0.0f);
        }
    }
    rs += __shfl_xor(rs, 32);
    if (half == 0 && valid) a.rsum[(size_t)rq * a.n_tiles + tile] = rs;
  }
}

// s_waitcnt on the vector-memory counter only: at most n loads of this wave
// may still be in flight (they complete in issue order).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define DSPARK_VMCNT(k) __builtin_amdgcn_s_waitcnt(((k) & 15) | (7 << 4) | (15 << 8) | (((k) >> 4) << 14))
  switch (n) {
    case 0: DSPARK_VMCNT(0); break;   case 1: DSPARK_VMCNT(1); break;   case 2: DSPARK_VMCNT(2); break;
    case 3: DSPARK_VMCNT(3); break;   case 4: DSPARK_VMCNT(4); break;   case 5: DSPARK_VMCNT(5); break;
    case 6: DSPARK_VMCNT(6); break;   case 7: DSPARK_VMCNT(7); break;   case 8: DSPARK_VMCNT(8); break;
    case 9: DSPARK_VMCNT(9); break;   case 10: DSPARK_VMCNT(10); break; case 11: DSPARK_VMCNT(11); break;
    case 12: DSPARK_VMCNT(12); break; case 13: DSPARK_VMCNT(13); break; case 14: DSPARK_VMCNT(14); break;
    case 15: DSPARK_VMCNT(15); break; case 16: DSPARK_VMCNT(16); break; case 20: DSPARK_VMCNT(20); break;
    case 24: DSPARK_VMCNT(24); break; case 32: DSPARK_VMCNT(32); break; case 36: DSPARK_VMCNT(36); break;
    case 40: DSPARK_VMCNT(40); break; case 48: DSPARK_VMCNT(48); break;
    default: DSPARK_VMCNT(0); break;
  }
#undef DSPARK_VMCNT
}

constexpr int kRing = 4;  // W2 tiles in flight: the fill of tile i+3 overlaps tiles i and i+1

template <typename TL, bool RESIDUAL, int R>
__global__ __launch_bounds__(512, 1) void gemm_stats_lds(GemmArgs a) {
  constexpr int KS = R / 16, NBLK = 2 * KS, TILE_BYTES = NBLK * 1024;
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
  // number of W2 operand blocks this wave loads per tile
  const int my_fills = (NBLK - wave + nwaves - 1) / nwaves;

  auto fill = [&](int tile, int buf) {
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
    // all operand reads of the tile are issued ahead in groups of four k-steps
    constexpr int GK = KS < 4 ? KS : 4;
    bf16x8 A[2][2][GK];
#pragma unroll
    for (int q = 0; q < GK; ++q)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) A[0][vb][q] = *reinterpret_cast<const bf16x8*>(base + (vb * KS + q) * 1024);
#pragma unroll
    for (int g = 0; g < KS / GK; ++g) {
      const int cur = g & 1;
      if (g + 1 < KS / GK) {
#pragma unroll
        for (int q = 0; q < GK; ++q)
#pragma unroll
          for (int vb = 0; vb < 2; ++vb)
            A[cur ^ 1][vb][q] = *reinterpret_cast<const bf16x8*>(base + (vb * KS + (g + 1) * GK + q) * 1024);
      }
#pragma unroll
      for (int q = 0; q < GK; ++q)
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[cur][vb][q], H[g * GK + q], acc[vb], 0, 0, 0);
    }
  };
  auto full_tile = [&](int tile) { return (tile + 1) * kTile <= V; };
  constexpr int kXLoads = 8;  // vector loads issued by load_tile()

  f32x16 acc0[2], acc1[2];
  TileBuf<TL> x0, x1;
  int t = blockIdx.x;
  // prologue: tiles t0..t2 requested, t0 computed
  fill(t, 0);
  if (t + G < nt) fill(t + G, 1);
  if (t + 2 * G < nt) fill(t + 2 * G, 2);
  if (active) load_tile<TL>(brow, t * kTile, half, V, x0);
  wait_vmcnt(0);
  __syncthreads();
  if (active) mma(0, acc0);

  // steady state, two tiles per trip so that accumulators and logit registers
  // are static; the W2 ring slot of tile t_i is i % kRing
  int i = 0;
  for (;;) {
    // tile t = t_i: acc0, x0; t_{i+1} ready in ring slot (i+1) % kRing
    int pending = 0;  // loads this wave issues in this iteration
    if (t + 3 * G < nt) fill(t + 3 * G, (i + 3) % kRing), pending += my_fills;
    if (t + G < nt && active) {
      load_tile<TL>(brow, (t + G) * kTile, half, V, x1);
      pending += kXLoads;
      mma((i + 1) % kRing, acc1);
    }
    if (active) epilogue_tile<TL, RESIDUAL>(a, acc0, x0, trow, rq, pos, valid, T, t, half, full_tile(t));
    wait_vmcnt(pending);  // the fill of t_{i+2} (issued one iteration ago) has landed
    __syncthreads();
    t += G, ++i;
    if (t >= nt) break;
    // tile t = t_i: acc1, x1; t_{i+1} ready in ring slot (i+1) % kRing
    pending = 0;
    if (t + 3 * G < nt) fill(t + 3 * G, (i + 3) % kRing), pending += my_fills;
    if (t + G < nt && active) {
      load_tile<TL>(brow, (t + G) * kTile, half, V, x0);
      pending += kXLoads;
      mma((i + 1) % kRing, acc0);
    }
    if (active) epilogue_tile<TL, RESIDUAL>(a, acc1, x1, trow, rq, pos, valid, T, t, half, full_tile(t));
    wait_vmcnt(pending);
    __syncthreads();
    t += G, ++i;
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
    if (((k1 - k0) & 7) == 0 && (k0 & 7) == 0 && k1 - k0 <= 64) {
      // every load first, then the products (one memory round trip)
      uint4 hv[8], wv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + 8 * i < k1) {
          hv[i] = *reinterpret_cast<const uint4*>(h + k0 + 8 * i);
          wv[i] = *reinterpret_cast<const uint4*>(w + k0 + 8 * i);
        }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (k0 + 8 * i < k1) {
          const uint32_t hh[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w}, ww[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
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

// Draw of block position `pos` for request b = blockIdx.x from the tile
// records (three-level exact Gumbel-max: block, tile, column), then the fp64
// recompute of the chosen tile for the token and its log-probability.
template <typename TL, typename TF>
__global__ __launch_bounds__(256) void draft_select_kernel(DraftSelectArgs a) {
  constexpr int kGroup = 64;  // blocks whose statistics are gathered per pass
  __shared__ double s_bm[kGroup], s_part[4][64];
  __shared__ float s_be[kGroup];
  __shared__ double s_val[4], s_lse;
  __shared__ int s_idx[4], s_tile;
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
    // wavefront 0, lane j: running choice and log-sum-exp over the groups
    double best = -INFINITY, row_m = -INFINITY, row_s = 0.0;
    int best_blk = 0x7fffffff;
    for (int g0 = 0; g0 < nblk; g0 += kGroup) {
      // Records of 4 chunks of 16 blocks, all requested at once: thread tid
      // holds tiles 4 tid .. 4 tid + 3 of each chunk, so the 16 lanes
      // 16 k .. 16 k + 15 of a wavefront hold one block, whose max and mass
      // (relative to that max) reduce within those lanes.
      double d[4][4];
      float sm[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = (g0 + 16 * q) * kTilesPerBlock + 4 * tid + k;
          if (t < nt) {
            const TileStat st = ts[t];
            d[q][k] = (double)st.ref + (double)st.mx, sm[q][k] = st.sum;
          } else {
            d[q][k] = -INFINITY, sm[q][k] = 0.0f;
          }
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double m = fmax(fmax(d[q][0], d[q][1]), fmax(d[q][2], d[q][3]));
        m = group16_max(m);
        float e = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (sm[q][k] > 0.0f) e += sm[q][k] * expf((float)((d[q][k] - m) * invT));
        e = group16_sum(e);
        const int j = 16 * q + 4 * wave + (lane >> 4);
        if ((lane & 15) == 0 && g0 + j < nblk) s_bm[j] = m, s_be[j] = e;
      }
      __syncthreads();
      if (wave == 0) {  // lane j: block g0 + j
        const int blk = g0 + lane;
        double val = -INFINITY, m = -INFINITY, e = 0.0;
        int idx = 0x7fffffff;
        if (blk < nblk) {
          m = s_bm[lane], e = (double)s_be[lane];
          val = (m - mref) * invT + log(e) + gumbel(a.seed, kDraftTop, b, rpos, blk);
          idx = blk;
        }
        wave_argmax(val, idx);
        if (val > best) best = val, best_blk = idx;  // groups in increasing order: ties keep the lowest
        const double gm = wave_max(m);
        const double gs = wave_sum(e > 0.0 ? e * exp((m - gm) * invT) : 0.0);
        if (gm > row_m) {
          row_s = row_s * exp((row_m - gm) * invT) + gs;
          row_m = gm;
        } else {
          row_s += gs * exp((gm - row_m) * invT);
        }
      }
      __syncthreads();
    }
    // tile inside the chosen block (its records were just read: an L2 hit)
    if (wave == 0) {
      const int blk = index_or(best_blk, nblk, 0);
      const int t0 = blk * kTilesPerBlock, t1 = min(t0 + kTilesPerBlock, nt);
      double val = -INFINITY;
      int ti = 0x7fffffff;
      if (t0 + lane < t1) {
        const TileStat st = ts[t0 + lane];
        val = ((double)st.ref + (double)st.mx - mref) * invT + log((double)st.sum) +
              gumbel(a.seed, kDraftMid, b, rpos, lane);
        ti = t0 + lane;
      }
      wave_argmax(val, ti);
      if (lane == 0) s_tile = index_or(ti, t1, t0), s_lse = row_m * invT + log(row_s);
    }
    __syncthreads();
    tile = s_tile, lse = s_lse;
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

  // recompute the chosen tile in fp64: the rank is split over the wavefronts;
  // the backbone logit is requested with the factor rows
  const int v = tile * kTile + lane;
  const double xb = (wave == 0 && v < V) ? (double)load_logit(brow + v) : 0.0;
  const int kq = (r + 3) / 4, k0 = min(wave * kq, r), k1 = min(k0 + kq, r);
  s_part[wave][lane] = v < V ? dot_part<TF>(h, Wt + (size_t)v * r, k0, k1) : 0.0;
  __syncthreads();
  if (wave == 0) {
    double lv = -INFINITY, sv = -INFINITY;
    int vi = 0x7fffffff;
    if (v < V) {
      const double d = xb + ((s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]));
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

// ---------------------------------------------------------------------------
// Coalesced draft kernel for bf16 logits (V a multiple of 8) and bf16 factors.
// A workgroup of 8 wavefronts owns 256 slots (32 per wavefront, the MFMA B
// operand columns, with their U rows held in registers) and walks the tiles
// t = blockIdx.x, + gridDim.x, ...  Both streams of a tile, the W2 rows and the
// backbone logits of the 256 slots, reach LDS by direct loads of whole rows
// into two-slot rings (layouts below); one barrier per tile.
// ---------------------------------------------------------------------------
// Reductions with the partner lane (lane ^ 32), identical in both lanes.
__device__ __forceinline__ float pair_max(float v) { return reduce_pair32(v, OpMax{}); }
__device__ __forceinline__ float pair_sum(float v) { return reduce_pair32(v, OpSum{}); }

// LDS layouts of the streamed tiles.  Every direct load writes one contiguous
// 1 KB block from whole rows; inside a block the 16-byte chunks are ordered
// chunk-major, and the blocks are spaced so that the operand reads of 16
// consecutive lanes fall in distinct bank groups while every lane's address for
// chunk c is its own base plus a constant (an instruction immediate).
//   W2 tile (64 rows x R bf16): RB = 1024 / (2R) rows per block, row rho's
//   chunk c at byte 16 (RB c + rho) of block b = row / RB, blocks 1024 + 16 RB
//   bytes apart.
//   logit tile (slots x 64 bf16): 8 slots per block, slot rho's chunk c at byte
//   16 (8 c + rho); block b starts at 1024 b + 8 (b % 2) + 128 ((b / 2) % 2)
//   + 256 (b / 4), so that 32 lanes' 8-byte reads of one chunk are disjoint.
template <int R>
struct WLayout {
  static constexpr int RB = 1024 / (2 * R);
  static constexpr int NB = kTile / RB;
  static constexpr int STRIDE = 1024 + 16 * RB;
  static constexpr int BYTES = NB * STRIDE;
  __device__ static int block(int b) { return b * STRIDE; }
  // byte offset of row v, chunk c
  __device__ static int at(int v, int c) { return (v / RB) * STRIDE + 16 * (RB * c + v % RB); }
};
struct XLayout {
  __device__ static int block(int b) { return b * 1024 + 8 * (b & 1) + 128 * ((b >> 1) & 1) + 256 * (b >> 2); }
  static constexpr int bytes(int slots) { return (slots / 8) * 1024 + 136 + 256 * (slots / 32); }
  __device__ static int at(int s, int c) { return block(s >> 3) + 16 * (8 * c + (s & 7)); }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int R>
__global__ __launch_bounds__(512, 1) void gemm_draft_coalesced(GemmArgs a) {
  using WL = WLayout<R>;
  constexpr int W_SLOT = (WL::BYTES + 1023) / 1024 * 1024;
  constexpr int X_SLOT = (XLayout::bytes(kSlotsPerGroup) + 1023) / 1024 * 1024;
  constexpr int KS = R / 16;                     // MFMA k-steps per tile
  constexpr int W_DMA = WL::NB / 8;              // direct loads per wave per tile: W2
  constexpr int X_DMA = kSlotsPerGroup / 64;     // and backbone logits
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  char* const wring = lds;                        // 2 x W_SLOT
  char* const xring = lds + 2 * W_SLOT;           // 2 x X_SLOT
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nslots = a.B;
  const int sg0 = blockIdx.y * kSlotsPerGroup;
  const int nt = a.n_tiles, G = gridDim.x;
  if (sg0 >= nslots || (int)blockIdx.x >= nt) return;  // uniform across the workgroup
  const int V = a.V;
  // byte offsets from uniform bases are 32-bit (the launcher checks the sizes)
  const char* const Wb = static_cast<const char*>(a.Wt);
  const char* const Xb = static_cast<const char*>(a.base);

  // direct load k of this wave for the W2 tile `tile` into ring slot buf
  auto dma_w = [&](int k, int tile, int buf) {
    const int f = wave + 8 * k;
    const int rho = lane % WL::RB, c = lane / WL::RB;
    const int v = min(tile * kTile + f * WL::RB + rho, V - 1);  // rows beyond V only feed masked columns
    __builtin_amdgcn_global_load_lds(Wb + ((uint32_t)v * (R * 2) + c * 16),
                                     (lds_ptr_t)(wring + buf * W_SLOT + WL::block(f)), 16, 0, 0);
  };
  // W2 needs nothing from the slots: the first two tiles start loading at once
  int t = blockIdx.x;
#pragma unroll
  for (int k = 0; k < W_DMA; ++k) dma_w(k, t, 0);
  if (t + G < nt) {
#pragma unroll
    for (int k = 0; k < W_DMA; ++k) dma_w(k, t + G, 1);
  }

  // this wave's 32 slots (MFMA B operand columns)
  const bool active = sg0 + wave * 32 < nslots;
  int rq, pos, prev;
  bool valid;
  slot_info<false>(a, sg0 + wave * 32 + l32, nslots, rq, pos, prev, valid);
  // backbone-logit rows this lane loads: slot 8 f + lane % 8 of the direct loads
  // f = wave + 8 k
  uint32_t xoff[X_DMA];  // element offset of the row in the backbone logits [B * gamma, V]
#pragma unroll
  for (int k = 0; k < X_DMA; ++k) {
    const int sx = (wave + 8 * k) * 8 + (lane & 7);
    int b2, p2, pr2;
    bool v2;
    slot_info<false>(a, sg0 + sx, nslots, b2, p2, pr2, v2);
    xoff[k] = (uint32_t)(b2 * a.gamma + p2) * (uint32_t)V;
  }
  auto dma_x = [&](int k, int tile, int buf) {
    const int f = wave + 8 * k;
    const int col = min(tile * kTile + ((lane >> 3) << 3), V - 8);  // the ragged tile is masked later
    __builtin_amdgcn_global_load_lds(Xb + (xoff[k] + col) * 2,
                                     (lds_ptr_t)(xring + buf * X_SLOT + XLayout::block(f)), 16, 0, 0);
  };
#pragma unroll
  for (int k = 0; k < X_DMA; ++k) dma_x(k, t, 0);

  const float T = valid ? effective_temp(a.temperature[rq]) : 1.0f;
  const float cT = T > 0.0f ? kLog2e / T : 0.0f;
  bf16x8 H[KS];
  {
    const uint16_t* h = static_cast<const uint16_t*>(a.U) + (size_t)prev * R + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 zero = {};
      H[ks] = valid ? *reinterpret_cast<const bf16x8*>(h + ks * 16) : zero;
    }
  }
  // operand bases: W2 row l32 (column block 0) with chunk half; logits of this
  // lane's slot, 8-byte half
  const int wbase = WL::at(l32, half);
  const int xbase = XLayout::at(wave * 32 + l32, 0) + 8 * half;
  const uint32_t st_base = (uint32_t)rq * (uint32_t)nt;

  auto read_x = [&](int buf, TileBuf<uint16_t>& x) {
    const char* p = xring + buf * X_SLOT + xbase;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 u = *reinterpret_cast<const uint2*>(p + 128 * (vb * 4 + g));
        x.w[vb][2 * g] = u.x, x.w[vb][2 * g + 1] = u.y;
      }
  };
  // streaming store of a tile record (nothing reads it before the next launch)
  auto put = [&](int tile, const TileStat& st) {
    const f32x4 v = {st.ref, st.mx, st.sum, 0.0f};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(reinterpret_cast<char*>(a.tstat) +
                                                            (st_base + (uint32_t)tile) * 16u));
  };
  // MFMAs of the next tile (W2 slot wb) interleaved by hand with the statistics
  // of the current one: k-step ks reads the operands of step ks + 1, issues its
  // two MFMAs and one slice of the epilogue, fenced so that the MFMA pipe and
  // the VALU work side by side within the wave.  The epilogue's phases (unpack
  // and tile max of the logits; t = (x - ref) + bias and its max; exp2 sum)
  // take the first, second and last two quarters of the k-steps.
  auto fused = [&](auto masked, int wb, int tile, const f32x16 (&cur)[2], f32x16 (&next)[2],
                   const TileBuf<uint16_t>& x, TileStat& st) {
    constexpr bool MASK = decltype(masked)::value;
    const char* base = wring + wb * W_SLOT + wbase;
    auto rd = [&](int ks, int vb) {  // rows vb * 32 + l32, chunk 2 ks + half
      return *reinterpret_cast<const bf16x8*>(base + 32 * WL::RB * ks + (32 / WL::RB) * WL::STRIDE * vb);
    };
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) next[i][e] = 0.0f;
    float xv[32];  // element j = 16 vb + e; becomes t in place
    float ref = -INFINITY, tmax = -INFINITY, mc = 0.0f, sum = 0.0f;
    bf16x8 A[2][2];
    A[0][0] = rd(0, 0), A[0][1] = rd(0, 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cb = ks & 1;
      if (ks + 1 < KS) A[cb ^ 1][0] = rd(ks + 1, 0), A[cb ^ 1][1] = rd(ks + 1, 1);
      next[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[cb][0], H[ks], next[0], 0, 0, 0);
      next[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[cb][1], H[ks], next[1], 0, 0, 0);
      constexpr int PA = KS / 4, PB = KS / 2;  // phase boundaries
      if (ks < PA) {
        constexpr int n = 32 / PA;
#pragma unroll
        for (int j = ks * n; j < ks * n + n; ++j) {
          const int vb = j >> 4, e = j & 15;
          xv[j] = x.get(vb, e);
          if (MASK && acc_col(tile * kTile, vb, e, half) >= V) xv[j] = -INFINITY;
          ref = fmaxf(ref, xv[j]);
        }
        asm volatile("" : "+v"(ref));  // keeps this slice in its k-step
      } else if (ks < PB) {
        if (ks == PA) ref = pair_max(ref);
        constexpr int n = 32 / (PB - PA);
#pragma unroll
        for (int j = (ks - PA) * n; j < (ks - PA) * n + n; ++j) {
          xv[j] = (xv[j] - ref) + cur[j >> 4][j & 15];
          tmax = fmaxf(tmax, xv[j]);
        }
        asm volatile("" : "+v"(tmax));  // keeps this slice in its k-step
      } else {
        if (ks == PB) tmax = pair_max(tmax), mc = tmax * cT;
        constexpr int n = 32 / (KS - PB);
#pragma unroll
        for (int j = (ks - PB) * n; j < (ks - PB) * n + n; ++j) sum += __builtin_amdgcn_exp2f(fmaf(xv[j], cT, -mc));
        asm volatile("" : "+v"(sum));  // keeps this slice in its k-step
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    st.ref = ref, st.mx = tmax, st.sum = pair_sum(sum), st.pad = 0.0f;
  };

  f32x16 acc0[2] = {}, acc1[2] = {};
  TileStat st;
  int st_tile = -1;
  wait_vmcnt(0);
  __syncthreads();
  if (active) {
    TileBuf<uint16_t> none = {};
    fused(std::false_type{}, 0, t, acc1, acc0, none, st);  // MFMAs of the first tile only
  }
  __syncthreads();
  // Ring discipline: in iteration i (tile t_i) W2 slot i%2, last read by the
  // MFMAs of t_i, receives W2 of t_{i+2}; logit slot (i+1)%2, emptied at the top
  // of iteration i-1, receives the logits of t_{i+1}.  The logits of t_i leave
  // LDS and the record of t_{i-1} goes out before any load is issued.
  auto step = [&](int c0, const f32x16 (&cur)[2], f32x16 (&next)[2]) {
    const int c1 = c0 ^ 1;
    TileBuf<uint16_t> x;
    if (active) {
      read_x(c0, x);
      if (st_tile >= 0 && half == 0 && valid) put(st_tile, st);
    }
    if (t + 2 * G < nt) {
#pragma unroll
      for (int k = 0; k < W_DMA; ++k) dma_w(k, t + 2 * G, c0);
    }
    if (t + G < nt) {
#pragma unroll
      for (int k = 0; k < X_DMA; ++k) dma_x(k, t + G, c1);
    }
    if (active) {
      // the MFMAs of the last tile's successor read a stale slot and are discarded
      if ((t + 1) * kTile <= V) fused(std::false_type{}, c1, t, cur, next, x, st);
      else fused(std::true_type{}, c1, t, cur, next, x, st);
      st_tile = t;
    }
    wait_vmcnt(0);
    __syncthreads();
    t += G;
  };
  for (;;) {
    step(0, acc0, acc1);
    if (t >= nt) break;
    step(1, acc1, acc0);
    if (t >= nt) break;
  }
  if (active && st_tile >= 0 && half == 0 && valid) put(st_tile, st);
}

template <int R>
hipError_t launch_coalesced(const GemmArgs& a, hipStream_t s) {
  static int max_wg = 0;
  const size_t lds = (size_t)2 * ((WLayout<R>::BYTES + 1023) / 1024 * 1024) +
                     (size_t)2 * ((XLayout::bytes(kSlotsPerGroup) + 1023) / 1024 * 1024);
  const void* fn = reinterpret_cast<const void*>(&gemm_draft_coalesced<R>);
  if (!max_wg) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorUnknown;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return hipErrorUnknown;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 512, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    max_wg = cus * per_cu;
  }
  const int groups = (a.B + kSlotsPerGroup - 1) / kSlotsPerGroup;
  const int wg_x = max(1, min(a.n_tiles, max_wg / groups));
  gemm_draft_coalesced<R><<<dim3(wg_x, groups), 512, lds, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Residual pass over bf16 logits (V a multiple of 8): for every request whose
// draft token at row n was rejected, the mass of max(0, p - q) in each tile,
// with q the draft distribution of row n recomputed from the backbone logits
// and the Markov bias.
//
// 128 slots per workgroup of 8 wavefronts: wavefront w holds the 32 slots
// 32 (w % 4) .. and computes column block w / 4 (32 columns) of every tile, 16
// MFMAs per tile.  The W2 tile (32 KB at R = 256), the backbone logits and the
// target logits of the 128 slots (16 KB each) stream through two-slot LDS rings
// by whole-row direct loads, swizzled as in the draft kernel; the two column
// halves of a slot's tile mass meet in a small LDS exchange.  Workgroups map to
// slot groups at run time from the device-side count of pending requests, so
// the whole grid works whatever that count is.
// ---------------------------------------------------------------------------
constexpr int kResSlots = 128;

template <int R>
__global__ __launch_bounds__(512, 1) void gemm_residual_coalesced(GemmArgs a) {
  constexpr int NC = R / 8;
  constexpr int W_BYTES = kTile * R * 2;
  constexpr int X_BYTES = kResSlots * kTile * 2;  // 16 KB
  constexpr int W_INSTR = W_BYTES / 1024, X_INSTR = X_BYTES / 1024;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  __shared__ float part[2][kResSlots];
  char* const wring = lds;                  // 2 x W_BYTES
  char* const xring = lds + 2 * W_BYTES;    // 2 x X_BYTES backbone logits
  char* const zring = xring + 2 * X_BYTES;  // 2 x X_BYTES target logits
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int vb = wave >> 2, sl = (wave & 3) * 32 + l32;  // column block, slot in the group
  const int nslots = (int)*a.slot_count;
  if (nslots <= 0) return;
  const int ngroups = (nslots + kResSlots - 1) / kResSlots;
  // walkers per slot group, a multiple of 8 so that the workgroups of one tile
  // share an XCD (and its L2) across groups
  int walkers = (int)gridDim.x / ngroups;
  if (walkers >= 8) walkers &= ~7;
  if (walkers < 1) walkers = 1;
  const int group = (int)blockIdx.x / walkers;
  const int nt = a.n_tiles, V = a.V;
  if (group >= ngroups || (int)blockIdx.x - group * walkers >= nt) return;  // uniform
  const int sg0 = group * kResSlots;
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);

  int rq, pos, prev;
  bool valid;
  slot_info<true>(a, sg0 + sl, nslots, rq, pos, prev, valid);
  const bool active = sg0 + (wave & 3) * 32 < nslots;
  float T = 1.0f, kp = 0.0f;
  double lse_q = 0.0;
  if (valid) {
    T = effective_temp(a.temperature[rq]);
    const ReqState st = a.req[rq];
    kp = (float)(((double)st.row_max / (double)T + st.row_logsum) * 1.4426950408889634);
    lse_q = a.draft_lse[(size_t)rq * a.gamma + pos];
  }
  if (!(T > 0.0f)) T = 1.0f;  // greedy rows never hold a residual draw
  const float c = kLog2e / T;
  bf16x8 H[R / 16];
  {
    const uint16_t* h = static_cast<const uint16_t*>(a.U) + (size_t)prev * R + half * 8;
#pragma unroll
    for (int ks = 0; ks < R / 16; ++ks) {
      const bf16x8 zero = {};
      H[ks] = valid ? *reinterpret_cast<const bf16x8*>(h + ks * 16) : zero;
    }
  }
  // rows this lane loads for the logit streams: slot f * 8 + lane / 8 of
  // instructions f = wave, wave + 8
  const uint16_t* xsrc[X_INSTR / 8];
  const uint16_t* zsrc[X_INSTR / 8];
#pragma unroll
  for (int k = 0; k < X_INSTR / 8; ++k) {
    const int sx = (wave + 8 * k) * 8 + (lane >> 3);
    int b2, p2, pr2;
    bool v2;
    slot_info<true>(a, sg0 + sx, nslots, b2, p2, pr2, v2);
    xsrc[k] = static_cast<const uint16_t*>(a.base) + ((size_t)b2 * a.gamma + p2) * V;
    zsrc[k] = static_cast<const uint16_t*>(a.target) + ((size_t)b2 * (a.gamma + 1) + p2) * V;
  }

  auto fill_w = [&](int tile, int buf) {
#pragma unroll
    for (int k = 0; k < W_INSTR / 8; ++k) {
      const int f = wave + 8 * k;
      const int r = f * (64 / NC) + lane / NC, p = lane % NC;
      int v = tile * kTile + r;
      v = v < V ? v : V - 1;  // rows beyond V only feed masked columns
      __builtin_amdgcn_global_load_lds(Wt + (size_t)v * R + (p ^ (r % NC)) * 8,
                                       (lds_ptr_t)(wring + buf * W_BYTES + f * 1024), 16, 0, 0);
    }
  };
  auto fill_xz = [&](int tile, int buf) {
#pragma unroll
    for (int k = 0; k < X_INSTR / 8; ++k) {
      const int f = wave + 8 * k;
      const int sx = f * 8 + (lane >> 3), p = lane & 7;
      const int col = min(tile * kTile + ((p ^ ((sx >> 1) & 7)) << 3), V - 8);  // ragged tile masked later
      __builtin_amdgcn_global_load_lds(xsrc[k] + col, (lds_ptr_t)(xring + buf * X_BYTES + f * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(zsrc[k] + col, (lds_ptr_t)(zring + buf * X_BYTES + f * 1024), 16, 0, 0);
    }
  };
  auto mma = [&](int buf, f32x16& acc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    const char* base = wring + buf * W_BYTES;
    const int v = vb * 32 + l32;
    auto rd = [&](int ks) {
      return *reinterpret_cast<const bf16x8*>(base + v * (R * 2) + (((2 * ks + half) ^ (v % NC)) << 4));
    };
    bf16x8 A[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) A[0][q] = rd(q);
#pragma unroll
    for (int g = 0; g < R / 64; ++g) {
      const int cur = g & 1;
      if (g + 1 < R / 64) {
#pragma unroll
        for (int q = 0; q < 4; ++q) A[cur ^ 1][q] = rd((g + 1) * 4 + q);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[cur][q], H[g * 4 + q], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // this lane's 16 columns of the tile: vb * 32 + 8 g + 4 half + (0..3), g = 0..3
  auto read_logits = [&](const char* ring, int buf, uint2 (&out)[4]) {
    const char* rowp = ring + buf * X_BYTES + sl * 128 + half * 8;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      out[g] = *reinterpret_cast<const uint2*>(rowp + (((vb * 4 + g) ^ ((sl >> 1) & 7)) << 4));
  };
  auto unpack = [](const uint2 (&w)[4], float (&v)[16]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v[4 * g + 0] = __uint_as_float(w[g].x << 16);
      v[4 * g + 1] = __uint_as_float(w[g].x & 0xFFFF0000u);
      v[4 * g + 2] = __uint_as_float(w[g].y << 16);
      v[4 * g + 3] = __uint_as_float(w[g].y & 0xFFFF0000u);
    }
  };
  auto epilogue = [&](const f32x16& acc, const uint2 (&xw)[4], const uint2 (&zw)[4], int tile) {
    float xv[16], zv[16];
    unpack(xw, xv);
    unpack(zw, zv);
    if ((tile + 1) * kTile > V) {  // the ragged last tile: columns >= V do not exist
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (tile * kTile + vb * 32 + (e >> 2) * 8 + half * 4 + (e & 3) >= V) xv[e] = -INFINITY, zv[e] = -INFINITY;
    }
    float ref = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) ref = fmaxf(ref, xv[e]);
    ref = reduce_pair32(ref, OpMax{});
    ref = ref > -INFINITY ? ref : 0.0f;  // a half tile wholly beyond V
    const float kq = (float)((lse_q - (double)ref / (double)T) * 1.4426950408889634);
    float rs = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(zv[e], c, -kp));
      const float q = __builtin_amdgcn_exp2f(fmaf((xv[e] - ref) + acc[e], c, -kq));
      rs += fmaxf(p - q, 0.0f);
    }
    return reduce_pair32(rs, OpSum{});
  };

  const int G = walkers;
  int t = (int)blockIdx.x - group * walkers;
  f32x16 acc0, acc1;
  fill_w(t, 0);
  if (t + G < nt) fill_w(t + G, 1);
  fill_xz(t, 0);
  wait_vmcnt(0);
  __syncthreads();
  if (active) mma(0, acc0);
  __syncthreads();
  // Ring discipline as in the draft kernel: in iteration i (tile t_i) W2 slot
  // i%2 receives W2 of t_{i+2} and logit slot (i+1)%2 the logits of t_{i+1};
  // the logits of t_i leave LDS first, before any load is in flight.
  auto step = [&](int c0, f32x16& cur, f32x16& next) {
    const int c1 = c0 ^ 1;
    uint2 xw[4], zw[4];
    if (active) read_logits(xring, c0, xw), read_logits(zring, c0, zw);
    if (t + 2 * G < nt) fill_w(t + 2 * G, c0);
    if (t + G < nt) fill_xz(t + G, c1);
    if (t + G < nt && active) mma(c1, next);
    float rs = 0.0f;
    if (active) {
      rs = epilogue(cur, xw, zw, t);
      if (vb == 1 && half == 0) part[c0][sl] = rs;
    }
    wait_vmcnt(0);
    __syncthreads();
    if (vb == 0 && half == 0 && valid) a.rsum[(size_t)rq * nt + t] = rs + part[c0][sl];
    t += G;
  };
  for (;;) {
    step(0, acc0, acc1);
    if (t >= nt) break;
    step(1, acc1, acc0);
    if (t >= nt) break;
  }
}

template <int R>
hipError_t launch_residual_coalesced(const GemmArgs& a, hipStream_t s) {
  static int max_wg = 0;
  const size_t lds = (size_t)2 * (kTile * R * 2) + (size_t)4 * (kResSlots * kTile * 2);
  const void* fn = reinterpret_cast<const void*>(&gemm_residual_coalesced<R>);
  if (!max_wg) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorUnknown;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return hipErrorUnknown;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 512, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    max_wg = cus * per_cu;
  }
  // enough workgroups to give every CU one, and at least one per tile of every
  // possible slot group when the batch is small
  const int groups = (a.B + kResSlots - 1) / kResSlots;
  const int grid = max(8, min(max_wg, groups * a.n_tiles));
  gemm_residual_coalesced<R><<<grid, 512, lds, s>>>(a);
  return hipGetLastError();
}

template <typename TL, bool RESIDUAL, int R>
hipError_t launch_pipelined(const GemmArgs& a, hipStream_t s) {
  static int max_wg = 0;
  const size_t lds = (size_t)kRing * (2 * (R / 16) * 1024);
  const void* fn = reinterpret_cast<const void*>(&gemm_stats_lds<TL, RESIDUAL, R>);
  if (!max_wg) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorUnknown;
    if (lds > 64 * 1024 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
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
  if constexpr (sizeof(TL) == 2) {
    // the coalesced kernels address their inputs with 32-bit byte offsets
    const bool fits = (size_t)a.B * (a.gamma + 1) * a.V * 2 < (1ull << 32) &&
                      (size_t)a.V * a.r * 2 < (1ull << 32) && (size_t)a.B * a.n_tiles * 16 < (1ull << 32);
    if (factor_dtype == DSPARK_BF16 && a.V % 8 == 0 && a.V >= 64 && (a.r == 128 || a.r == 256) && fits) {
      if constexpr (RESIDUAL) {
        if (a.r == 256) return launch_residual_coalesced<256>(a, s);
        return launch_residual_coalesced<128>(a, s);
      } else {
        if (a.r == 256) return launch_coalesced<256>(a, s);
        return launch_coalesced<128>(a, s);
      }
    }
  }
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

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
    // blocks of this wavefront in chunks of 16: all tile records of a chunk are
    // requested first, then reduced block by block; lane j keeps block j's
    // (max, mass), and the 16 Gumbels and logarithms are computed in parallel
    for (int c0 = wave; c0 < nblk; c0 += 64) {
      TileStat rec[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = (c0 + 4 * j) * kTilesPerBlock + lane;
        if (c0 + 4 * j < nblk && t < nt) rec[j] = ts[t];
        else rec[j].ref = -INFINITY, rec[j].mx = 0.0f, rec[j].sum = 0.0f;
      }
      double my_d = -INFINITY, my_s = 0.0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + 4 * j >= nblk) break;  // uniform
        const double d = (double)rec[j].ref + (double)rec[j].mx;
        const double dmax = wave_max(d);
        const float e = rec[j].sum > 0.0f ? rec[j].sum * expf((float)((d - dmax) * invT)) : 0.0f;
        const float sblk = wave_sum(e);
        if (lane == j) my_d = dmax, my_s = (double)sblk;
      }
      const int blk = c0 + 4 * lane;
      if (lane < 16 && blk < nblk) {
        const double val = (my_d - mref) * invT + log(my_s) + gumbel(a.seed, kDraftTop, b, rpos, blk);
        if (val > best) best = val, best_blk = blk;
        if (my_d > row_m) {
          row_s = row_s * exp((row_m - my_d) * invT) + my_s;
          row_m = my_d;
        } else {
          row_s += my_s * exp((my_d - row_m) * invT);
        }
      }
    }
    wave_argmax(best, best_blk);
    {
      const double m = wave_max(row_m);
      row_s = wave_sum(row_s > 0.0 ? row_s * exp((row_m - m) * invT) : 0.0);
      row_m = m;
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

// ---------------------------------------------------------------------------
// Coalesced variant for bf16 logits (V a multiple of 8), the one the headline
// round runs.  Both streams of a tile go through LDS by direct loads whose every
// instruction reads whole rows:
//   * W2 tile: 64 rows x R bf16.  Instruction f reads 64/NC full rows (NC = R/8
//     16-byte chunks per row); lane l takes chunk (l % NC) ^ (row % NC) of its
//     row, so LDS holds the rows with their chunks xor-swizzled by the row and
//     the MFMA operand reads (32 rows, one chunk each) spread over all banks.
//   * backbone logits: 256 slots x 64 columns x 2 B; instruction f reads 8 full
//     128-byte slot rows, chunk (l % 8) ^ (slot % 8) per lane, swizzled alike
//     for the epilogue's 8-byte reads.
// Two-slot rings for both (128 KB of LDS at R = 256).
// ---------------------------------------------------------------------------
template <bool RESIDUAL, int R>
__global__ __launch_bounds__(512, 1) void gemm_stats_coalesced(GemmArgs a) {
  constexpr int NC = R / 8;                       // 16-byte chunks per W2 row
  constexpr int W_BYTES = kTile * R * 2;          // 32 KB at R = 256
  constexpr int X_BYTES = kSlotsPerGroup * kTile * 2;  // 32 KB
  constexpr int W_INSTR = W_BYTES / 1024, X_INSTR = X_BYTES / 1024;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  char* const wring = lds;                        // 2 x W_BYTES
  char* const xring = lds + 2 * W_BYTES;          // 2 x X_BYTES
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nslots = RESIDUAL ? (int)*a.slot_count : a.B;
  const int sg0 = blockIdx.y * kSlotsPerGroup;
  const int nt = a.n_tiles, G = gridDim.x;
  if (sg0 >= nslots || (int)blockIdx.x >= nt) return;  // uniform across the workgroup
  const int V = a.V;
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);

  // this wave's 32 slots (MFMA B operand columns)
  const bool active = sg0 + wave * 32 < nslots;
  int rq, pos, prev;
  bool valid;
  slot_info<RESIDUAL>(a, sg0 + wave * 32 + l32, nslots, rq, pos, prev, valid);
  const uint16_t* trow = RESIDUAL
      ? static_cast<const uint16_t*>(a.target) + ((size_t)rq * (a.gamma + 1) + pos) * V : nullptr;
  const float T = valid ? effective_temp(a.temperature[rq]) : 1.0f;
  bf16x8 H[R / 16];
  {
    const uint16_t* h = static_cast<const uint16_t*>(a.U) + (size_t)prev * R + half * 8;
#pragma unroll
    for (int ks = 0; ks < R / 16; ++ks) {
      const bf16x8 zero = {};
      H[ks] = valid ? *reinterpret_cast<const bf16x8*>(h + ks * 16) : zero;
    }
  }
  // rows of the backbone logits this lane loads for the logit stream: slot
  // f*8 + lane/8 of each of this wave's instructions f = wave, wave+nwaves, ...
  constexpr int XMAX = X_INSTR;  // at most one instruction per wave per 8 slots
  const uint16_t* xsrc[4];
  int nx = 0;
  for (int f = wave; f < X_INSTR && nx < 4; f += nwaves, ++nx) {
    const int s = f * 8 + (lane >> 3);
    int b2, p2, pr2;
    bool v2;
    slot_info<RESIDUAL>(a, sg0 + s, nslots, b2, p2, pr2, v2);
    xsrc[nx] = static_cast<const uint16_t*>(a.base) + ((size_t)b2 * a.gamma + p2) * V;
  }
  (void)XMAX;

  auto fill_w = [&](int tile, int buf) {
    for (int f = wave; f < W_INSTR; f += nwaves) {
      const int r = f * (64 / NC) + lane / NC, p = lane % NC;
      int v = tile * kTile + r;
      v = v < V ? v : V - 1;  // rows beyond V only feed masked columns
      const int c = p ^ (r % NC);
      __builtin_amdgcn_global_load_lds(Wt + (size_t)v * R + c * 8,
                                       (lds_ptr_t)(wring + buf * W_BYTES + f * 1024), 16, 0, 0);
    }
  };
  auto fill_x = [&](int tile, int buf) {
    int k = 0;
    for (int f = wave; f < X_INSTR && k < 4; f += nwaves, ++k) {
      const int s = f * 8 + (lane >> 3), p = lane & 7;
      const int c = p ^ (s & 7);
      const int col = min(tile * kTile + c * 8, V - 8);  // the ragged tile is masked later
      __builtin_amdgcn_global_load_lds(xsrc[k] + col, (lds_ptr_t)(xring + buf * X_BYTES + f * 1024), 16, 0, 0);
    }
  };
  auto mma = [&](int buf, f32x16 (&acc)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    const char* base = wring + buf * W_BYTES;
    bf16x8 A[2][2][4];
    auto rd = [&](int ks, int vb) {
      const int v = vb * 32 + l32, c = 2 * ks + half;
      return *reinterpret_cast<const bf16x8*>(base + v * (R * 2) + ((c ^ (v % NC)) << 4));
    };
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) A[0][vb][q] = rd(q, vb);
#pragma unroll
    for (int g = 0; g < R / 64; ++g) {
      const int cur = g & 1;
      if (g + 1 < R / 64) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) A[cur ^ 1][vb][q] = rd((g + 1) * 4 + q, vb);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[cur][vb][q], H[g * 4 + q], acc[vb], 0, 0, 0);
    }
  };
  auto read_x = [&](int buf, TileBuf<uint16_t>& x) {
    const int s = wave * 32 + l32;
    const char* rowp = xring + buf * X_BYTES + s * 128 + half * 8;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = vb * 4 + g;
        const uint2 u = *reinterpret_cast<const uint2*>(rowp + ((c ^ (s & 7)) << 4));
        x.w[vb][2 * g] = u.x, x.w[vb][2 * g + 1] = u.y;
      }
  };
  auto full_tile = [&](int tile) { return (tile + 1) * kTile <= V; };

  f32x16 acc0[2], acc1[2];
  int t = blockIdx.x;
  // Ring discipline: at the start of iteration i (tile t_i) the W2 slot i%2
  // (last read by the MFMAs of t_i in iteration i-1) receives W2 of t_{i+2}, and
  // the logit slot (i+1)%2 (last read by the epilogue of t_{i-1}) receives the
  // logits of t_{i+1}; both loads have the whole iteration to land.
  fill_w(t, 0);
  if (t + G < nt) fill_w(t + G, 1);
  fill_x(t, 0);
  wait_vmcnt(0);
  __syncthreads();
  if (active) mma(0, acc0);
  __syncthreads();

  int i = 0;
  for (;;) {
    // tile t = t_i with accumulators acc0
    {
      const int c0 = i & 1, c1 = c0 ^ 1;
      if (t + 2 * G < nt) fill_w(t + 2 * G, c0);
      if (t + G < nt) fill_x(t + G, c1);
      if (t + G < nt && active) mma(c1, acc1);
      if (active) {
        TileBuf<uint16_t> x;
        read_x(c0, x);
        epilogue_tile<uint16_t, RESIDUAL>(a, acc0, x, trow, rq, pos, valid, T, t, half, full_tile(t));
      }
      wait_vmcnt(0);
      __syncthreads();
      t += G, ++i;
      if (t >= nt) break;
    }
    // tile t = t_i with accumulators acc1
    {
      const int c0 = i & 1, c1 = c0 ^ 1;
      if (t + 2 * G < nt) fill_w(t + 2 * G, c0);
      if (t + G < nt) fill_x(t + G, c1);
      if (t + G < nt && active) mma(c1, acc0);
      if (active) {
        TileBuf<uint16_t> x;
        read_x(c0, x);
        epilogue_tile<uint16_t, RESIDUAL>(a, acc1, x, trow, rq, pos, valid, T, t, half, full_tile(t));
      }
      wait_vmcnt(0);
      __syncthreads();
      t += G, ++i;
      if (t >= nt) break;
    }
  }
}

template <bool RESIDUAL, int R>
hipError_t launch_coalesced(const GemmArgs& a, hipStream_t s) {
  static int max_wg = 0;
  const size_t lds = (size_t)2 * (kTile * R * 2) + (size_t)2 * (kSlotsPerGroup * kTile * 2);
  const void* fn = reinterpret_cast<const void*>(&gemm_stats_coalesced<RESIDUAL, R>);
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
  const int wg_x = max(1, min(a.n_tiles, max_wg / groups));
  gemm_stats_coalesced<RESIDUAL, R><<<dim3(wg_x, groups), 64 * kLdsWaves, lds, s>>>(a);
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
    if (factor_dtype == DSPARK_BF16 && a.V % 8 == 0 && a.V >= 64 && (a.r == 128 || a.r == 256)) {
      if (a.r == 256) return launch_coalesced<RESIDUAL, 256>(a, s);
      return launch_coalesced<RESIDUAL, 128>(a, s);
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

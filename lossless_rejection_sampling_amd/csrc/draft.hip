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

#include <atomic>
#include <type_traits>

#include "dspark.h"
#include "kernels.hpp"
#include "schedule_body.hpp"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLog2eD = 1.4426950408889634;

// Residual-mode passes serve two calls.  The residual draw: slots are the
// requests queued in slot_req[0..*slot_count), each at its rejected row, with the
// statistics of that target row in req[b]; a tile's value is the mass of
// max(0, p - q).  The acceptance pass (tv set): slot s is (request s / gamma,
// row s % gamma) for all B gamma of them, row statistics in rowinfo[s]; a tile's
// value is the mass of min(p, q).  Outputs go to rsum[(b or s) * n_tiles + tile].
__device__ __forceinline__ int residual_slots(const GemmArgs& a) {
  return a.tv ? a.B * a.gamma : (int)*a.slot_count;
}
__device__ __forceinline__ void residual_rowstats(const GemmArgs& a, int b, int pos, double& mx, double& lsum) {
  if (a.tv) {
    const double2 r = a.rowinfo[(size_t)b * a.gamma + pos];
    mx = r.x, lsum = r.y;
  } else {
    mx = a.req[b].row_max, lsum = a.req[b].row_logsum;
  }
}
__device__ __forceinline__ float residual_mass(const GemmArgs& a, float p, float q) {
  return a.tv ? fminf(p, q) : fmaxf(p - q, 0.0f);
}
__device__ __forceinline__ size_t residual_out(const GemmArgs& a, int b, int pos, int tile) {
  return (a.tv ? (size_t)b * a.gamma + pos : (size_t)b) * a.n_tiles + tile;
}

// Largest number of slots a launch must cover (host side).
inline int max_slots(const GemmArgs& a, bool residual) { return residual && a.tv ? a.B * a.gamma : a.B; }

// Which request, base row and previous token a GEMM slot stands for.
template <bool RESIDUAL>
__device__ __forceinline__ void slot_info(const GemmArgs& a, int s, int nslots, int& b, int& pos,
                                          int& prev, bool& valid) {
  valid = s < nslots;
  if (RESIDUAL) {
    if (a.tv) {
      b = valid ? s / a.gamma : 0;
      pos = valid ? s - b * a.gamma : 0;
    } else {
      b = valid ? a.slot_req[s] : 0;
      pos = valid ? a.req[b].n : 0;
    }
  } else {
    b = valid ? s : 0;
    pos = a.pos;
  }
  int pv = pos == 0 ? a.prev0[b] : a.draft[(size_t)b * a.gamma + pos - 1];
  prev = valid ? checked_token(pv, a.V, a.status, pos == 0 ? kBadPrev : kBadDraft) : 0;
}

// The draft tile record of the logit type (8 bytes for bf16 logits, whose t
// carries no shift; 16 for fp32, shifted by the tile's largest backbone logit).
template <typename TL>
__device__ __forceinline__ void put_rec(void* ts, size_t i, float ref, float mx, float sum) {
  if constexpr (sizeof(TL) == 2) {
    static_cast<TileStat*>(ts)[i] = TileStat{mx, sum};
  } else {
    static_cast<TileStatRef*>(ts)[i] = TileStatRef{ref, mx, sum, 0.0f};
  }
}
// Whether the draft statistics shift t by the tile's largest backbone logit
// (fp32 logits; the residual masses always do, since any shift serves them).
template <typename TL, bool RESIDUAL>
constexpr bool kShiftByTileMax = RESIDUAL || sizeof(TL) != 2;

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
  const int nslots = RESIDUAL ? residual_slots(a) : a.B;
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
    ref = kShiftByTileMax<TL, RESIDUAL> ? fmaxf(ref, __shfl_xor(ref, 32)) : 0.0f;  // the shift of t
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
      if (half == 0 && valid[bb]) put_rec<TL>(a.tstat, (size_t)rq * a.n_tiles + tile, ref, tmax, s);
    } else {
      // r(v) = max(0, p(v) - q(v)) with p from the target row and q rebuilt from
      // the draft statistics of the same position.
      float rs = 0.0f;
      if (valid[bb]) {
        double rmax, rlsum;
        residual_rowstats(a, rq, pos[bb], rmax, rlsum);
        const float invT = 1.0f / T;
        const float mp = (float)rmax, lsp = (float)rlsum;
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
              rs += residual_mass(a, p, q);
            }
          }
      }
      rs += __shfl_xor(rs, 32);
      if (half == 0 && valid[bb]) a.rsum[residual_out(a, rq, pos[bb], tile)] = rs;
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
  float ref = 0.0f;  // the shift of t
  if constexpr (kShiftByTileMax<TL, RESIDUAL>) {
    ref = -INFINITY;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 16; ++e) ref = fmaxf(ref, xv[vb][e]);
    ref = fmaxf(ref, __shfl_xor(ref, 32));
  }
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
    if (half == 0 && valid) put_rec<TL>(a.tstat, (size_t)rq * a.n_tiles + tile, ref, tmax, s);
  } else {
    TileBuf<TL> z;
    load_tile<TL>(trow, tile * kTile, half, a.V, z);
    float rs = 0.0f;
    if (valid) {
      double rmax, rlsum;
      residual_rowstats(a, rq, pos, rmax, rlsum);
      const float c = kLog2e / T;
      // p = 2^((z - max) c - ln S log2 e): the difference first (an exact input
      // value is subtracted), so no term carries an error proportional to max / T
      const float mz = (float)rmax, kp = (float)(rlsum * 1.4426950408889634);
      const double lse_q = a.draft_lse[(size_t)rq * a.gamma + pos];
      const float kq = (float)((lse_q - (double)ref / (double)T) * 1.4426950408889634);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float zv = (full || acc_col(tile * kTile, vb, e, half) < a.V) ? z.get(vb, e) : -INFINITY;
          const float p = __builtin_amdgcn_exp2f(fmaf(zv - mz, c, -kp));
          const float q = __builtin_amdgcn_exp2f(fmaf(t[vb][e], c, -kq));
          rs += residual_mass(a, p, q);
        }
    }
    rs += __shfl_xor(rs, 32);
    if (half == 0 && valid) a.rsum[residual_out(a, rq, pos, tile)] = rs;
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

template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

constexpr int kRing = 4;  // W2 tiles in flight: the fill of tile i+3 overlaps tiles i and i+1

template <typename TL, bool RESIDUAL, int R>
__global__ __launch_bounds__(512, 1) void gemm_stats_lds(GemmArgs a) {
  constexpr int KS = R / 16, NBLK = 2 * KS, TILE_BYTES = NBLK * 1024;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nslots = RESIDUAL ? residual_slots(a) : a.B;
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
  const int nslots = RESIDUAL ? residual_slots(a) : a.B;
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
  const float ref = kShiftByTileMax<TL, RESIDUAL> ? wave_max(x) : 0.0f;  // the shift of t
  const float t = ok ? (x - ref) + bias : -INFINITY;
  const float tmax = wave_max(t);
  const float T = effective_temp(a.temperature[b]);
  if constexpr (!RESIDUAL) {
    const float c = T > 0.0f ? kLog2e / T : 0.0f;
    const float sum = wave_sum(ok ? exp2f((t - tmax) * c) : 0.0f);
    if (lane == 0) put_rec<TL>(a.tstat, (size_t)b * a.n_tiles + tile, ref, tmax, sum);
  } else {
    double rmax, rlsum;
    residual_rowstats(a, b, pos, rmax, rlsum);
    const float invT = 1.0f / T;
    const double lse_q = a.draft_lse[(size_t)b * a.gamma + pos];
    const float cq = (float)(lse_q - (double)ref / (double)T);
    float rv = 0.0f;
    if (ok) {
      const TL* trow = static_cast<const TL*>(a.target) + ((size_t)b * (a.gamma + 1) + pos) * V;
      const float p = expf((load_logit(trow + v) - (float)rmax) * invT - (float)rlsum);
      const float q = expf(t * invT - cq);
      rv = residual_mass(a, p, q);
    }
    const float sum = wave_sum(rv);
    if (lane == 0) a.rsum[residual_out(a, b, pos, tile)] = sum;
  }
}

// Shift and mass of one block of 64 tiles held by 16 lanes (4 tiles a lane):
// e = sum_t S_t exp((d_t - m) / T) with the fp32 maximum of the d_t as the
// shift m.  Any shift near the largest d_t gives the same block value
// (m - ref) / T + log(e) up to rounding, and an fp32 maximum takes half the
// exchange steps of an fp64 one.  v_exp_f32 on the fp64 exponent rounded to
// fp32; terms below 2^-126 of the largest flush to zero.
__device__ __forceinline__ void block_mass(const double (&d)[4], const float (&sm)[4], double invT_log2e,
                                           double& m_out, float& e_out) {
  float mf = fmaxf(fmaxf((float)d[0], (float)d[1]), fmaxf((float)d[2], (float)d[3]));
  mf = group16_max(mf);
  const double m = (double)mf;
  float e = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (sm[k] > 0.0f) e += sm[k] * __builtin_amdgcn_exp2f((float)((d[k] - m) * invT_log2e));
  m_out = m, e_out = group16_sum(e);
}

// The row's log-sum-exp (lse, in units of logit / T) with the chosen tile's
// share of the row's mass taken from the tile's fp64 recompute (sv = d / T of
// each live lane's column) in place of its share from the tile record:
//   lse + log(1 - share_rec + share_exact).
// share_rec is the record's term exactly as the block sums included it
// (block_mass: the fp32 exponent of (d - m_blk) / T and v_exp_f32), relative to
// the row's shift gm and sum gs.  The record's top logit carries one fp32
// rounding at |t|'s scale, which 1/T magnifies; where the chosen tile holds
// most of the mass, this removes nearly all of it from ln q.
__device__ __forceinline__ double exact_tile_lse(double lse, double sv, bool live, double rec_d, float rec_sum,
                                                 double m_blk, double gm, double gs, double invT) {
  // both shares as v_exp_f32 of exponents formed in fp64 (relative error ~1e-7)
  const float e = live ? __builtin_amdgcn_exp2f((float)((sv - lse) * kLog2eD)) : 0.0f;
  const double ex = (double)wave_sum(e);
  float term = 0.0f;
  if (rec_sum > 0.0f) term = rec_sum * __builtin_amdgcn_exp2f((float)((rec_d - m_blk) * (invT * kLog2eD)));
  const double rec = (double)(term * __builtin_amdgcn_exp2f((float)((m_blk - gm) * invT * kLog2eD))) / gs;
  // the shares differ by the record's rounding only: log1p by its series
  const double d = ex - rec;
  return lse + (fabs(d) < 1e-3 ? d * (1.0 - d * (0.5 - d * (1.0 / 3.0))) : log1p(d));
}

// The copy of U[x] into the table the next position's contraction reads (only
// with bf16 factors at r = 128 or 256, one 16-byte chunk a lane): the load in
// the constructor, the store in store(), so that work placed between them runs
// while the load is in flight.
template <typename TF>
struct HrowCopy {
  uint4 u;
  bool on;
  __device__ __forceinline__ HrowCopy(const DraftSelectArgs& a, int b, int x, int pos, int lane) : u{}, on(false) {
    if constexpr (sizeof(TF) == 2) {
      on = a.hrows && pos + 1 < a.gamma && a.r <= 512 && lane * 8 < a.r;
      if (on) u = reinterpret_cast<const uint4*>(static_cast<const TF*>(a.U) + (size_t)x * a.r)[lane];
    }
  }
  __device__ __forceinline__ void store(const DraftSelectArgs& a, int b, int x, int lane) const {
    if constexpr (sizeof(TF) == 2) {
      if (on) reinterpret_cast<uint4*>(static_cast<TF*>(a.hrows) + (size_t)b * a.r)[lane] = u;
    }
  }
};

// ---------------------------------------------------------------------------
// One draw per request at block position pos+1 (a workgroup of 4 wavefronts
// per request): three-level Gumbel-max over blocks of 64 tiles, tiles of 64
// columns, and columns.  Block and tile levels use the tile statistics (one
// coalesced 512-byte read per block for bf16 logits, 1 KB for fp32); the chosen
// tile is recomputed in fp64 with
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
      // a product of two bf16 values (8-bit significands) is exact in fp32; the
      // sum runs in fp64 over four independent chains
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
  const TileRec<TL>* ts = static_cast<const TileRec<TL>*>(a.tstat) + (size_t)b * nt;
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * gamma + pos) * V;
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;
  const TF* Wt = static_cast<const TF*>(a.Wt);
  const int nblk = (nt + kTilesPerBlock - 1) / kTilesPerBlock;

  int tile;  // chosen tile
  double invT = 0.0, lse = 0.0;
  double row_m = -INFINITY, row_s = 0.0;            // wavefront 0: the row's shift and sum
  double c_mblk = 0.0, c_d = 0.0;                   // wavefront 0: the chosen block's shift, the tile's top logit
  float c_sum = 0.0f;                               // and its exp-sum
  if (Tf > 0.0f) {
    invT = 1.0 / (double)Tf;
    const double mref = rec_top(ts[0]);
    // wavefront 0, lane j: running choice and log-sum-exp over the groups
    double best = -INFINITY;
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
            const TileRec<TL> st = ts[t];
            d[q][k] = rec_top(st), sm[q][k] = st.sum;
          } else {
            d[q][k] = -INFINITY, sm[q][k] = 0.0f;
          }
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double m;
        float e;
        block_mass(d[q], sm[q], invT * kLog2eD, m, e);
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
      double val = -INFINITY, d = -INFINITY;
      float sm = 0.0f;
      int ti = 0x7fffffff;
      if (t0 + lane < t1) {
        const TileRec<TL> st = ts[t0 + lane];
        d = rec_top(st), sm = st.sum;
        val = (d - mref) * invT + log((double)st.sum) + gumbel(a.seed, kDraftMid, b, rpos, lane);
        ti = t0 + lane;
      }
      // the block's shift as block_mass takes it: the fp32 maximum of its tiles' top logits
      c_mblk = (double)wave_max((float)d);
      wave_argmax(val, ti);
      const int chosen = index_or(ti, t1, t0);
      c_d = __shfl(d, chosen - t0), c_sum = __shfl(sm, chosen - t0);
      if (lane == 0) s_tile = chosen, s_lse = row_m * invT + log(row_s);
    }
    __syncthreads();
    tile = s_tile, lse = s_lse;
  } else {
    double best = -INFINITY;
    int bt = 0x7fffffff;
    for (int t = tid; t < nt; t += 256) {
      const double d = rec_top(ts[t]);
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
    HrowCopy<TF> cp(a, b, x, pos, lane);  // requested before the log-sum-exp's last step
    if (Tf > 0.0f) lse = exact_tile_lse(lse, sv, v < V, c_d, c_sum, c_mblk, row_m, row_s, invT);
    if (lane == 0) {
      a.draft[(size_t)b * gamma + pos] = x;
      a.logq[(size_t)b * gamma + pos] = Tf > 0.0f ? (float)(sx - lse) : 0.0f;
      a.lse[(size_t)b * gamma + pos] = Tf > 0.0f ? lse : sx;
    }
    cp.store(a, b, x, lane);
  }
}

// Draw of block position `pos` for request b = blockIdx.x when the row has at
// most 64 blocks (V <= 262144): the same three-level draw and fp64 recompute
// as draft_select_kernel with three memory round trips on the critical path.
//   1. The tile records, the temperature and the previous token are requested
//      together; meanwhile waves 0, 1 and 2 compute the block-, tile- and
//      column-level Gumbel values of this draw (they depend on no data).
//   2. Records go to LDS; 16-lane groups reduce each block; wave 0 draws the
//      block, then the tile from the LDS copy, while wave 1 forms the row's
//      log-sum-exp.
//   3. The chosen tile is recomputed in fp64 (bf16 factors at r = 128 or 256:
//      eight lanes a factor row, whole lines per load, the U[prev] chunks
//      requested in step 1; otherwise the rank split over the four
//      wavefronts), the column drawn, and U[x] copied for the next position.
// The arithmetic of every value that decides a draw is that of
// draft_select_kernel, up to the order of the fp64 sums of exact products.
constexpr int kDrawMaxTiles = kTilesPerBlock * 64;
struct DrawShared {
  double d[kDrawMaxTiles];   // largest draft logit of every tile
  float sum[kDrawMaxTiles];  // exp-sum of every tile
  double g[3][64];           // Gumbel values: block, tile, column level
  double bm[64], part[4][64];
  float be[64];
  double val[8], lse, gm, gs;
  int idx[8], tile;
};

// Accesses to data that other workgroups of the same launch write or read
// (agent-scope relaxed atomics: coherent across the XCDs' L2 caches).
__device__ __forceinline__ TileStat load_rec_coherent(const TileStat* p) {
  const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return TileStat{__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32))};
}
__device__ __forceinline__ void store_rec_coherent(TileStat* p, float mx, float sum) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)__float_as_uint(mx) | ((uint64_t)__float_as_uint(sum) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// COHERENT: the tile records and the previous position's token were written by
// other workgroups of the same launch, and the token drawn here is read by them.
// NW: wavefronts of the workgroup (4 or 8).  Each 16-lane group covers the same
// 64 tiles of a block and each factor row of the recompute is summed by the
// same 8 lanes either way, so the results do not depend on NW.
template <typename TL, typename TF, bool COHERENT = false, int NW = 4>
__device__ __forceinline__ void draft_select_block(const DraftSelectArgs& a, int b, DrawShared& sh) {
  static_assert(NW == 4 || NW == 8, "four or eight wavefronts");
  constexpr int NQ = 16 / NW;     // groups of four tiles per lane
  constexpr int QS = 256 * NW;    // tiles per group: tile QS q + 4 tid + k

  auto& s_d = sh.d;
  auto& s_sum = sh.sum;
  auto& s_g = sh.g;
  auto& s_bm = sh.bm;
  auto& s_part = sh.part;
  auto& s_be = sh.be;
  auto& s_val = sh.val;
  auto& s_lse = sh.lse;
  auto& s_idx = sh.idx;
  auto& s_tile = sh.tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V, r = a.r, gamma = a.gamma, nt = a.n_tiles, pos = a.pos;
  const int nblk = (nt + kTilesPerBlock - 1) / kTilesPerBlock;
  using Rec = TileRec<TL>;
  static_assert(!COHERENT || sizeof(TL) == 2, "coherent records are the bf16 kind");
  const Rec* ts = static_cast<const Rec*>(a.tstat) + (size_t)b * nt;

  // 1. every load of the draw's first phase at once
  const float T_raw = a.temperature[b];
  const int prev_raw = pos == 0                 ? a.prev0[b]
                       : COHERENT               ? load_coherent(a.draft + (size_t)b * gamma + pos - 1)
                                                : a.draft[(size_t)b * gamma + pos - 1];
  const uint32_t off = a.pos_offset ? (uint32_t)a.pos_offset[b] : 0u;
  Rec rec[NQ][4];  // tiles QS q + 4 tid + k (unconditional loads, so that they all go out at once)
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const Rec* p = ts + min(QS * q + 4 * tid + k, nt - 1);
      if constexpr (COHERENT) rec[q][k] = load_rec_coherent(p);
      else rec[q][k] = *p;
    }
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (QS * q + 4 * tid + k >= nt) rec[q][k].mx = -INFINITY, rec[q][k].sum = 0.0f;
  const uint32_t rpos = (uint32_t)(pos + 1) + off;
  if (wave < 3 && (wave != 0 || lane < nblk)) s_g[wave][lane] = gumbel(a.seed, kDraftTop + wave, b, rpos, lane);
  const float Tf = checked_temp(T_raw, a.status);
  const int prev = checked_token(prev_raw, V, a.status, pos == 0 ? kBadPrev : kBadDraft);
  const TF* h = static_cast<const TF*>(a.U) + (size_t)prev * r;

  // 2. records to LDS; block statistics over 16-lane groups
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = QS * q + 4 * tid + k;
      if (t < nt) s_d[t] = rec_top(rec[q][k]), s_sum[t] = rec[q][k].sum;
    }
  int tile;
  double lse = 0.0;
  if (Tf > 0.0f) {
    const double invT = 1.0 / (double)Tf;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      double d[4], m;
      float sm[4], e;
#pragma unroll
      for (int k = 0; k < 4; ++k) d[k] = rec_top(rec[q][k]), sm[k] = rec[q][k].sum;
      block_mass(d, sm, invT * kLog2eD, m, e);
      const int j = (QS / kTilesPerBlock) * q + 4 * wave + (lane >> 4);
      if ((lane & 15) == 0 && j < nblk) s_bm[j] = m, s_be[j] = e;
    }
    __syncthreads();
    if (wave == 1) {
      // the row's log-sum-exp, beside the draw
      double m = -INFINITY, e = 0.0;
      if (lane < nblk) m = s_bm[lane], e = (double)s_be[lane];
      const double gm = wave_max(m);
      const double gs = wave_sum(e > 0.0 ? e * exp((m - gm) * invT) : 0.0);
      if (lane == 0) s_lse = gm * invT + log(gs), sh.gm = gm, sh.gs = gs;
    } else if (wave == 0) {
      const double mref = s_d[0];
      // block (lane j)
      double val = -INFINITY;
      int idx = 0x7fffffff;
      if (lane < nblk) {
        val = (s_bm[lane] - mref) * invT + log((double)s_be[lane]) + s_g[0][lane];
        idx = lane;
      }
      wave_argmax(val, idx);
      // tile inside the chosen block
      const int blk = index_or(idx, nblk, 0);
      const int t0 = blk * kTilesPerBlock, t1 = min(t0 + kTilesPerBlock, nt);
      double tv = -INFINITY;
      int ti = 0x7fffffff;
      if (t0 + lane < t1) {
        tv = (s_d[t0 + lane] - mref) * invT + log((double)s_sum[t0 + lane]) + s_g[1][lane];
        ti = t0 + lane;
      }
      wave_argmax(tv, ti);
      if (lane == 0) s_tile = index_or(ti, t1, t0);
    }
    __syncthreads();
    tile = s_tile, lse = s_lse;
  } else {
    // greedy: the tile with the largest logit (lowest index on ties)
    double best = -INFINITY;
    int bt = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = QS * q + 4 * tid + k;
        const double d = rec_top(rec[q][k]);
        if (t < nt && d > best) best = d, bt = t;
      }
    wave_argmax(best, bt);
    if (lane == 0) s_val[wave] = best, s_idx[wave] = bt;
    __syncthreads();
    best = -INFINITY, bt = 0x7fffffff;
    for (int w = 0; w < NW; ++w)
      if (s_val[w] > best || (s_val[w] == best && s_idx[w] < bt)) best = s_val[w], bt = s_idx[w];
    tile = index_or(bt, nt, 0);
  }

  // 3. fp64 recompute of the chosen tile (bf16 factors at r = 128 or 256: its
  // U[prev] chunks and W rows in one round trip; requested any earlier, these
  // conditional loads make the compiler's waits for the tile records wait for
  // them too)
  TileDot td;
  td.nj = sizeof(TF) == 2 && (r == 128 || r == 256) ? r / 64 : 0;
  if (td.nj) td.load_h(reinterpret_cast<const uint16_t*>(h), lane);
  const TL* brow = static_cast<const TL*>(a.base) + ((size_t)b * gamma + pos) * V;
  const int v = tile * kTile + lane;
  const float xb = load_logit(brow + min(v, V - 1));  // unconditional: issued with the factor rows
  if (td.nj) {
    double dt[2];
    td.dot<8 / NW>(static_cast<const uint16_t*>(a.Wt), tile * kTile, V, wave, lane, dt);
    if ((lane & 7) == 0) {
      s_part[0][(64 / NW) * wave + (lane >> 3)] = dt[0];
      if (NW == 4) s_part[0][(64 / NW) * wave + (lane >> 3) + 8] = dt[1];
    }
  } else if (wave < 4) {
    // the rank split over four wavefronts
    const int kq = (r + 3) / 4, k0 = min(wave * kq, r), k1 = min(k0 + kq, r);
    s_part[wave][lane] = v < V ? dot_part<TF>(h, static_cast<const TF*>(a.Wt) + (size_t)v * r, k0, k1) : 0.0;
  }
  __syncthreads();
  if (wave == 0) {
    double lv = -INFINITY, sv = -INFINITY;
    int vi = 0x7fffffff;
    if (v < V) {
      const double dot = td.nj ? s_part[0][lane] : (s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]);
      const double d = (double)xb + dot;
      if (Tf > 0.0f) {
        sv = d / (double)Tf;
        lv = sv + s_g[2][lane];
      } else {
        sv = d;
        lv = d;
      }
      vi = v;
    }
    wave_argmax(lv, vi);
    const int x = index_or(vi, min(V, (tile + 1) * kTile), tile * kTile);
    const double sx = __shfl(sv, x - tile * kTile);
    // U[x] for the next position's contraction is requested first; the
    // log-sum-exp's last step runs while it is in flight
    HrowCopy<TF> cp(a, b, x, pos, lane);
    if (Tf > 0.0f) {
      const int blk = tile / kTilesPerBlock;
      lse = exact_tile_lse(lse, sv, v < V, s_d[tile], s_sum[tile], s_bm[blk], sh.gm, sh.gs, 1.0 / (double)Tf);
    }
    if (lane == 0) {
      if (COHERENT)
        __hip_atomic_store(a.draft + (size_t)b * gamma + pos, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        a.draft[(size_t)b * gamma + pos] = x;
      a.logq[(size_t)b * gamma + pos] = Tf > 0.0f ? (float)(sx - lse) : 0.0f;
      a.lse[(size_t)b * gamma + pos] = Tf > 0.0f ? lse : sx;
    }
    cp.store(a, b, x, lane);
  }
}

// Eight wavefronts: the block sums and the records' LDS copies, on one
// wavefront per SIMD with every latency exposed, are split twice as finely.
template <typename TL, typename TF>
__global__ __launch_bounds__(512) void draft_select_fast(DraftSelectArgs a) {
  __shared__ DrawShared sh;
  draft_select_block<TL, TF, false, 8>(a, blockIdx.x, sh);
}

// The last draw of a round and the scheduler (independent of each other, both
// bound by memory latency) in one launch: the first workgroups are the
// scheduler's, the last B draw.
struct SelectScheduleArgs {
  DraftSelectArgs d;
  ScheduleArgs s;
};

template <typename TL, typename TF>
__global__ __launch_bounds__(256) void draft_select_schedule(SelectScheduleArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ DrawShared sh;
  // the scheduler's workgroups come first: its chain of phases is the longer
  // one, and the dispatcher reaches low workgroup indices first
  const int ns = (int)gridDim.x - a.d.B;
  if ((int)blockIdx.x < ns) schedule_block(a.s, (int)blockIdx.x, ns, smem);
  else draft_select_block<TL, TF>(a.d, (int)blockIdx.x - ns, sh);
}

// ---------------------------------------------------------------------------
// Streaming draft kernel for bf16 logits (V a multiple of 8) and bf16 factors,
// R in {128, 256}.  A workgroup of 8 wavefronts owns 256 slots (32 per
// wavefront: the MFMA B operand columns, whose gathered rows U[prev] stay in
// registers) and walks the 64-column tiles t = blockIdx.x + j * gridDim.x, each
// as two 32-column stages (half-tiles).
//
//  * Column order.  MFMA row i of a stage stands for column perm(i) of its 32,
//    perm(8 g + 4 h + q) = 16 h + 4 g + q, so the 16 accumulator elements a
//    lane holds for its slot are 16 consecutive columns.
//  * Both streams reach LDS by direct loads into four-stage rings, three
//    stages ahead: the stage's W2 rows (shared by the workgroup, stored in MFMA
//    row order with the bank-spreading layout WLayout) and each wavefront's own
//    32 backbone-logit rows (64 bytes each, private to the wavefront).  No
//    register is ever the target of an outstanding load inside the loop, and
//    every wait is explicit.
//  * The accumulator sums the bias alone (it starts at zero, so its roundings
//    are at the bias's scale); the epilogue forms t = x + bias with one
//    rounding (a bf16 logit is exact in fp32).  With no shift to carry, a tile
//    record is (max t, exp-sum): 8 bytes.
//  * Iteration u issues the MFMAs of stage u+1 interleaved with the
//    statistics of stage u; the two stages of a tile are merged into one
//    record; the wait at the end covers only the loads of stage u+2.
// ---------------------------------------------------------------------------
// Reductions with the partner lane (lane ^ 32), identical in both lanes.
__device__ __forceinline__ float pair_max(float v) { return reduce_pair32(v, OpMax{}); }
__device__ __forceinline__ float pair_sum(float v) { return reduce_pair32(v, OpSum{}); }

// LDS layout of a streamed block of W2 rows (ROWS rows x R bf16).  Every direct
// load writes one contiguous 1 KB block from whole rows; inside a block the
// 16-byte chunks are ordered chunk-major, and the blocks are spaced so that the
// operand reads of 16 consecutive lanes fall in distinct bank groups while every
// lane's address for chunk c is its own base plus a constant (an instruction
// immediate): RB = 1024 / (2R) rows per block, row s's chunk c at byte
// 16 (RB c + s % RB) of block s / RB, blocks 1024 + 16 RB bytes apart.
template <int R, int ROWS = kTile>
struct WLayout {
  static constexpr int RB = 1024 / (2 * R);
  static constexpr int NB = ROWS / RB;
  static constexpr int STRIDE = 1024 + 16 * RB;
  static constexpr int BYTES = NB * STRIDE;
  __device__ static int block(int b) { return b * STRIDE; }
  // byte offset of row s, chunk c
  __device__ static int at(int s, int c) { return (s / RB) * STRIDE + 16 * (RB * c + s % RB); }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Column (within a 32-column stage) of MFMA row i.
__device__ __forceinline__ int col_of_row(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

// Workgroup barrier without a memory fence (the waits before it are explicit).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kStages = 4;      // ring depth (stages of 32 columns)
constexpr int kStageCols = 32;
constexpr int kXStageBytes = 32 * kStageCols * 2;  // one wavefront's logits of a stage: 2 KB

template <int R>
__global__ __launch_bounds__(512, 1) void gemm_draft_stream(GemmArgs a) {
  using WL = WLayout<R, kStageCols>;
  constexpr int KS = R / 16;                  // MFMA k-steps per stage
  constexpr int W_DMA = WL::NB / 8;           // direct loads per wave per stage: W2
  constexpr int X_DMA = kXStageBytes / 1024;  // and this wave's backbone logits
  constexpr int W_RING = kStages * WL::BYTES;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nslots = a.B;
  const int sg0 = blockIdx.y * kSlotsPerGroup;
  const int nt = a.n_tiles, G = gridDim.x;
  if (sg0 >= nslots || (int)blockIdx.x >= nt) return;  // uniform across the workgroup
  const int V = a.V;
  char* const xring = lds + W_RING + wave * (kStages * kXStageBytes);  // this wave's logit ring
  // byte offsets from uniform bases are 32-bit (the launcher checks the sizes)
  const char* const Wb = static_cast<const char*>(a.Wt);
  const char* const Xb = static_cast<const char*>(a.base);

  // Tiles of this workgroup.  Workgroups are dealt to the 8 XCDs round robin
  // (blockIdx.x % 8), each XCD with its own L2.  In the nt / G full rounds the
  // G tiles of a round are split into 8 runs of G / 8 adjacent tiles, one per
  // XCD, so the 8-byte records of neighbouring tiles of a row meet in one L2
  // and leave it as whole lines.  The nt % G leftover tiles go to the workgroups
  // of even XCDs first (odd XCDs stream measurably slower in this kernel).
  // Without a multiple of 8 workgroups the order is plain: tile bx + j G.
  const int bx = blockIdx.x, full = nt / G, rem = nt - full * G;
  const bool xcd_order = (G & 7) == 0;
  const int run_pos = xcd_order ? (bx & 7) * (G >> 3) + (bx >> 3) : bx;
  const int tail_rank = xcd_order ? (bx & 1) * (G >> 1) + (bx >> 1) : bx;
  auto tile_of = [&](int j) { return j < full ? j * G + run_pos : full * G + tail_rank; };
  // Stage u: tile tile_of(u / 2), columns 32 (u % 2) onwards; stages past the
  // last one repeat it (their loads hit L2 and their results are never used), so
  // every iteration issues the same loads.
  const int n_stage = 2 * (full + (tail_rank < rem ? 1 : 0));
  if (n_stage == 0) return;  // no tile (only with more workgroups than tiles)
  auto stage_col = [&](int u) {
    u = min(u, n_stage - 1);
    return tile_of(u >> 1) * kTile + (u & 1) * kStageCols;
  };
  auto dma_w = [&](int u, int slot) {
    const int c0 = stage_col(u);
#pragma unroll
    for (int k = 0; k < W_DMA; ++k) {
      const int f = wave + 8 * k;
      const int s = f * WL::RB + lane % WL::RB, c = lane / WL::RB;
      const int v = min(c0 + col_of_row(s), V - 1);  // rows >= V feed masked columns
      __builtin_amdgcn_global_load_lds(Wb + ((uint32_t)v * (R * 2) + c * 16),
                                       (lds_ptr_t)(lds + slot * WL::BYTES + WL::block(f)), 16, 0, 0);
    }
  };
  // this wave's 32 slots (request = slot, row = block position a.pos); lanes
  // without a valid slot work on row 0 and write their records to the spare row B
  // (any number of lanes may write it: its contents are never read)
  const int slot = sg0 + wave * 32 + l32;
  const bool valid = slot < nslots;
  const int rq = valid ? slot : 0;
  const uint32_t xrow = (uint32_t)(rq * a.gamma + a.pos) * (uint32_t)V;  // element offset of the slot's row
  // Backbone logits: direct load k, lane L fetches chunk 2k + L / 32 (8 columns)
  // of slot L % 32's row, so lane (half, l32) later reads its 32 bytes (columns
  // 16 half .. + 15) as chunks at k = half, L = l32 and L = 32 + l32.
  auto dma_x = [&](int u, int slot) {
    const int c0 = stage_col(u);
#pragma unroll
    for (int k = 0; k < X_DMA; ++k) {
      const int col = min(c0 + (2 * k + half) * 8, V - 8);  // the ragged stage is masked later
      __builtin_amdgcn_global_load_lds(Xb + (xrow + (uint32_t)col) * 2u,
                                       (lds_ptr_t)(xring + slot * kXStageBytes + k * 1024), 16, 0, 0);
    }
  };
  const uint32_t st_spare = (uint32_t)nslots * (uint32_t)nt;
  const uint32_t st_base = valid ? (uint32_t)rq * (uint32_t)nt : st_spare;
  auto store_rec = [&](uint32_t at, float mx, float sum) {
    const float2 rec = {mx, sum};  // TileStat
    // an ordinary store: the line stays in L2 until the neighbouring records
    // of the same XCD's run have joined it, and leaves as a whole line
    *reinterpret_cast<float2*>(reinterpret_cast<char*>(a.tstat) + at * 8u) = rec;
  };

  // The temperature and the U rows of the previous tokens (from the table the
  // previous draw filled, or gathered through prev0 at position 0) are loaded
  // and waited for before any stream load: the compiler's wait for a register
  // load issued before pending direct-to-LDS loads drains those too.  Then
  // the stream loads, in the order (vmcnt counts in issue order)
  //   W(0), X(0), W(1), X(1), W(2), X(2), W(3), X(3) | W(4), X(4) |
  //   W(5), X(5), record | W(6), X(6) | ...
  const float T_raw = a.temperature[rq];
  bf16x8 H[KS];
  {
    const uint16_t* h;
    if (a.hrows) {
      h = static_cast<const uint16_t*>(a.hrows) + (size_t)rq * R;
    } else {
      const int p0 = a.prev0[rq];
      h = static_cast<const uint16_t*>(a.U) + (size_t)(valid ? checked_token(p0, V, a.status, kBadPrev) : 0) * R;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) H[ks] = *reinterpret_cast<const bf16x8*>(h + half * 8 + ks * 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0070 | (0xF << 8));  // vmcnt(0): T and the U rows have landed
  const float T = valid ? effective_temp(T_raw) : 1.0f;
  const float cT = T > 0.0f ? kLog2e / T : 0.0f;
  __builtin_amdgcn_sched_barrier(0);
  dma_w(0, 0);
  dma_x(0, 0);
  dma_w(1, 1);
  dma_x(1, 1);
  dma_w(2, 2);
  dma_x(2, 2);
  dma_w(3, 3);
  dma_x(3, 3);

  const int wbase = WL::at(l32, half);          // operand base: storage row l32, chunk half
  const int xbase = half * 1024 + l32 * 16;     // this lane's first logit chunk in a stage

  // the accumulator of a stage starts at zero: it sums the bias alone, at the
  // bias's own scale
  auto seed = [&](f32x16& acc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  };
  // this lane's 16 backbone logits of stage slot `slot`
  auto read_x = [&](int slot, float (&x)[16]) {
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(xring + slot * kXStageBytes + xbase);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(xring + slot * kXStageBytes + xbase + 512);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t w = e < 8 ? w0[(e & 7) >> 1] : w1[(e & 7) >> 1];
      x[e] = (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
  };
  // operand of k-step ks: storage row l32, chunk 2 ks + half of the W2 stage in ring slot `slot`
  auto rd = [&](int slot, int ks) {
    return *reinterpret_cast<const bf16x8*>(lds + slot * WL::BYTES + wbase + 32 * WL::RB * ks);
  };
  // MFMAs of the next stage (ring slot `slot`, accumulator `next`, already
  // seeded) interleaved with the statistics of the current stage (`cur` holds
  // t): max over the first quarter of the k-steps, exp2-sum over the next half.
  auto fused = [&](int slot, const f32x16& cur, f32x16& next, float& tmax, float& sum) {
    tmax = -INFINITY, sum = 0.0f;
    float mc = 0.0f;
    bf16x8 A[2];
    A[0] = rd(slot, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) A[(ks + 1) & 1] = rd(slot, ks + 1);
      next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks & 1], H[ks], next, 0, 0, 0);
      constexpr int PA = KS / 4, PB = PA + KS / 2;  // phase boundaries
      if (ks < PA) {
        constexpr int n = 16 / PA;
#pragma unroll
        for (int j = ks * n; j < ks * n + n; ++j) tmax = fmaxf(tmax, cur[j]);
        asm volatile("" : "+v"(tmax));  // keeps this slice in its k-step
      } else if (ks < PB) {
        if (ks == PA) tmax = pair_max(tmax), mc = tmax * cT;
        constexpr int n = 16 / (PB - PA);
#pragma unroll
        for (int j = (ks - PA) * n; j < (ks - PA) * n + n; ++j)
          sum += __builtin_amdgcn_exp2f(fmaf(cur[j], cT, -mc));
        asm volatile("" : "+v"(sum));  // keeps this slice in its k-step
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sum = pair_sum(sum);
  };

  // Iteration u (stage u in ring slot S = u % 4 has its bias in `cur`; stage
  // u+1 in slot S+1 has landed):
  //   take stage u's backbone logits from slot S (t = x + bias, one
  //   rounding); seed `next` for stage u+1; issue stage u+4 into slot S; run the
  //   MFMAs of stage u+1 with the statistics of stage u; on a tile's second
  //   stage (odd u) merge with the first and store the record; wait for stage
  //   u+2, issued in iteration u-2 (or in the prologue), barrier.  The loads
  //   of iterations u-1 and u (2 (W_DMA + X_DMA)) are younger than X(u+2) and
  //   may stay in flight.  Record stores are not counted: a store may complete
  //   before older loads, so counting it could let the wait pass early, while
  //   leaving it out only ever waits longer.
  int jt = 0, tile = tile_of(0);
  float mx_first = 0.0f, sum_first = 0.0f;
  auto step = [&](auto S_, f32x16& cur, f32x16& next, int u) {
    constexpr int S = decltype(S_)::value;
    constexpr bool second = S & 1;  // stage u is the second half of its tile
    float x[16];
    read_x(S, x);
    seed(next);
    // slot S is rewritten below: its logits must have reached registers
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_w(u + 4, S);
    dma_x(u + 4, S);
#pragma unroll
    for (int e = 0; e < 16; ++e) cur[e] = x[e] + cur[e];
    const int c0 = tile * kTile + (second ? kStageCols : 0);
    if (c0 + kStageCols > V) {  // a ragged stage: columns >= V do not exist
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (c0 + half * 16 + e >= V) cur[e] = -INFINITY;
    }
    float mx, sum;
    fused((S + 1) % kStages, cur, next, mx, sum);
    if (second) {
      // merge the tile's two stages (a stage wholly beyond V has sum 0)
      const float m = fmaxf(mx_first, mx);
      float s = sum_first * __builtin_amdgcn_exp2f((mx_first - m) * cT);
      if (sum > 0.0f) s += sum * __builtin_amdgcn_exp2f((mx - m) * cT);
      if (half == 0) store_rec(st_base + (uint32_t)tile, m, s);  // both halves hold the same values
      tile = tile_of(++jt);
    } else {
      mx_first = mx, sum_first = sum;
    }
    wait_vmcnt_c<2 * (W_DMA + X_DMA)>();
    barrier_only();
  };

  f32x16 acc0, acc1;
  // prologue: stage 0 landed (the loads of stages 1 to 3 may be pending)
  wait_vmcnt_c<3 * (W_DMA + X_DMA)>();
  barrier_only();
  seed(acc0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd(0, ks), H[ks], acc0, 0, 0, 0);
  wait_vmcnt_c<2 * (W_DMA + X_DMA)>();  // stage 1 landed
  barrier_only();  // ... in every wave, and every wave is done with ring slot 0
  // steady state, unrolled four times so that ring slots are immediates
  for (int u = 0;; u += 4) {
    step(std::integral_constant<int, 0>{}, acc0, acc1, u + 0); if (u + 1 >= n_stage) break;
    step(std::integral_constant<int, 1>{}, acc1, acc0, u + 1); if (u + 2 >= n_stage) break;
    step(std::integral_constant<int, 2>{}, acc0, acc1, u + 2); if (u + 3 >= n_stage) break;
    step(std::integral_constant<int, 3>{}, acc1, acc0, u + 3); if (u + 4 >= n_stage) break;
  }
}

template <int R>
hipError_t launch_draft_stream(const GemmArgs& a, hipStream_t s) {
  const size_t lds = (size_t)kStages * (WLayout<R, kStageCols>::BYTES + 8 * kXStageBytes);
  int max_wg = 0;
  const hipError_t e = kernel_setup(reinterpret_cast<const void*>(&gemm_draft_stream<R>), 512, lds, &max_wg);
  if (e != hipSuccess) return e;
  const int groups = (a.B + kSlotsPerGroup - 1) / kSlotsPerGroup;
  const int wg_x = max(1, min(a.n_tiles, max_wg / groups));
  launch(&gemm_draft_stream<R>, dim3(wg_x, groups), 512, lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Resident draft round (bf16 logits, bf16 factors, r = 256): one cooperative
// launch of one workgroup per CU runs every block position of the round, so
// that W2 crosses the memory system once per round instead of once per
// position.
//
//  * Ownership.  Workgroup c owns the contiguous tiles [c nt / G, (c+1) nt / G)
//    for the whole round; their 2 x (tiles) 32-column stages are split into
//    contiguous runs over the 4 wavefronts (one per SIMD, 512 registers each),
//    at most kResStagesPerWave = 5 a wavefront.  A wavefront's W2 stages stay
//    in registers (AGPRs and VGPRs) as MFMA A operands: 5 x 16 k-steps x 4 =
//    320 registers; MFMA row i of a stage stands for column col_of_row(i), as
//    in the streaming kernel, so a lane's 16 accumulators are 16 consecutive
//    columns of its slot.
//  * A position.  Slot groups of 32 requests in turn: the U rows of the group
//    (gathered through the previous tokens) and each wavefront's backbone rows
//    of its stages arrive in LDS by direct loads two groups ahead; per stage
//    16 MFMAs with the U rows as B operand, then the tile statistics exactly as
//    in the streaming kernel (t = x + bias, max, exp2-sum).  Stage
//    statistics meet in LDS, where the workgroup merges the two stages of each
//    tile into the tile's record.
//  * Between phases.  The records of a position (all workgroups) feed the
//    draws; the tokens drawn feed the next position's gather.  Both cross
//    workgroups as agent-scope relaxed atomics (coherent across the XCDs' L2
//    caches without write-back or invalidation of the caches), and each phase
//    ends with a device-wide wait: every wavefront waits for its own stores
//    (vmcnt(0)), the workgroup raises its flag to the phase number, and one
//    wavefront polls all flags.  The poll is bounded in time; when the bound
//    passes (only if the workgroups were not all resident) the kStall bit is
//    set and the kernel runs on to its end.  The last workgroup out resets the
//    flags, so they are zero between calls.
//  * The draw of request b runs in workgroup b mod G with draft_select_block's
//    arithmetic, so the round's results are those of the per-position launches.
// ---------------------------------------------------------------------------
constexpr int kResWaves = 4;
constexpr int kResStagesPerWave = 5;  // W2 stages (32 columns x 256) held in registers per wavefront
constexpr int kResMaxB = 2048;        // requests (their tokens and temperatures live in LDS)
constexpr int kResMaxGrid = 1024;     // workgroups (phase flags in the workspace)
// Backbone rows of a slot group: the workgroup's 32 rows x (8 x tiles) 16-byte
// chunks, row-major with rows padded to an odd number of chunks (so that the
// reads of 16 consecutive rows at one column fall in distinct banks), loaded by
// row-contiguous direct loads (each 1 KB instruction covers one or two rows).
constexpr int kResXInstr = 11;  // direct loads per wavefront and slot group: 4 x 11 KB >= 32 x 81 chunks
constexpr int kResXBufBytes = kResWaves * kResXInstr * 1024;
constexpr int kResRingBytes = 2 * kResXBufBytes;  // two slot groups

struct ResidentGemmShared {
  uint4 urows[2][32 * 32];                          // U rows of two slot groups, 16-byte chunks swizzled
  float2 st[2][kResWaves * kResStagesPerWave + 1][32];  // (max, exp-sum) per stage and slot; the last row is a sink
  int32_t tok[kResMaxB];                             // previous token of every request
};
constexpr size_t kResUnionBytes =
    sizeof(ResidentGemmShared) > sizeof(DrawShared) ? sizeof(ResidentGemmShared) : sizeof(DrawShared);
// ... then the exp2 scale of every request
constexpr size_t kResLdsBytes = kResRingBytes + ((kResUnionBytes + 15) & ~(size_t)15) + kResMaxB * sizeof(float);

// Eight bf16 -inf values: the backbone chunks past V load this instead, so the
// columns that do not exist enter the statistics as t = -inf with no masking.
__device__ const uint4 kNegInfChunk = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};

struct ResidentArgs {
  DraftSelectArgs d;
  uint32_t* flags;      // [gridDim.x] phase reached by each workgroup (zero between calls)
  uint32_t* exits;      // workgroups finished (zero between calls)
  uint64_t spin_limit;  // bound of a device-wide wait, in s_memrealtime ticks (100 MHz)
};

// LDS stores written as instructions of their own: the compiler would otherwise
// wait for every direct-to-LDS load in flight (vmcnt(0)) before a store that it
// cannot prove disjoint from their targets.  Only for LDS that no direct load
// writes; completion is covered by the caller's lgkmcnt wait.
__device__ __forceinline__ void lds_store_f32x2(float2* p, float x, float y) {
  const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(p);
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(make_float2(x, y)) : "memory");
}

// The LDS reads of one tile record's merge (two stage statistics and the slot's
// exp2 scale), issued together and waited for in the same block, likewise
// without the compiler's wait for direct loads in flight.
__device__ __forceinline__ void lds_load_record_parts(const float2* p0, const float2* p1, const float* pc,
                                                      float2& s0, float2& s1, float& c) {
  const uint32_t a0 = (uint32_t)reinterpret_cast<uintptr_t>(p0), a1 = (uint32_t)reinterpret_cast<uintptr_t>(p1);
  const uint32_t ac = (uint32_t)reinterpret_cast<uintptr_t>(pc);
  asm volatile(
      "ds_read_b64 %0, %3\n\t"
      "ds_read_b64 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s0), "=&v"(s1), "=&v"(c)
      : "v"(a0), "v"(a1), "v"(ac)
      : "memory");
}

// Device-wide wait for phase `phase`.  The caller has waited for its own stores.
__device__ __forceinline__ void grid_phase(const ResidentArgs& ra, uint32_t phase) {
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(ra.flags + blockIdx.x, phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x < 64) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      int done = 1;
      for (int i = threadIdx.x; i < (int)gridDim.x; i += 64)
        done &= __hip_atomic_load(ra.flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= phase;
      if (__all(done)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > ra.spin_limit) {
        if (threadIdx.x == 0) flag_status(ra.d.status, kStall);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256, 1) void draft_round_resident(ResidentArgs ra) {
  constexpr int R = 256, KS = R / 16, KW = kResStagesPerWave;
  constexpr int X_DMA = kResXInstr;  // direct loads of backbone rows per wavefront and slot group
  constexpr int U_DMA = 4;       // and of U rows (16 KB per group over 4 wavefronts)
  const DraftSelectArgs& a = ra.d;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  ResidentGemmShared& gs = *reinterpret_cast<ResidentGemmShared*>(lds + kResRingBytes);
  DrawShared& dsh = *reinterpret_cast<DrawShared*>(lds + kResRingBytes);
  float* const cTs = reinterpret_cast<float*>(lds + kResRingBytes + ((kResUnionBytes + 15) & ~(size_t)15));
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: everything derived from it is scalar
  const int G = gridDim.x, cu = blockIdx.x;
  const int B = a.B, gamma = a.gamma, V = a.V, nt = a.n_tiles;
  const int NG = (B + 31) / 32;
  const int T0 = (int)((long long)cu * nt / G), T1 = (int)((long long)(cu + 1) * nt / G);
  const int ntl = T1 - T0, ns = 2 * ntl;
  const int S0 = wave * ns / kResWaves, S1 = (wave + 1) * ns / kResWaves, nsw = S1 - S0;
  // backbone buffer rows: 8 ntl chunks and one of padding
  const uint32_t nch = 8u * (uint32_t)ntl, rs = nch + 1u, rs_magic = 0xFFFFFFFFu / rs + 1u;
  const char* const Wb = static_cast<const char*>(a.Wt);
  const char* const Xb = static_cast<const char*>(a.base);
  const char* const Ub = static_cast<const char*>(a.U);

  for (int b = tid; b < B; b += 256) {
    const float T = effective_temp(a.temperature[b]);
    cTs[b] = T > 0.0f ? kLog2e / T : 0.0f;
  }

  // W2 stages into registers (rows >= V read row V - 1: their columns are masked)
  bf16x8 Wr[KW][KS];
#pragma unroll
  for (int i = 0; i < KW; ++i) {
    const int c0 = (2 * T0 + S0 + min(i, max(nsw - 1, 0))) * kStageCols;
    const int v = max(min(c0 + col_of_row(l32), V - 1), 0);
    const char* p = Wb + (size_t)v * (R * 2) + half * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Wr[i][ks] = *reinterpret_cast<const bf16x8*>(p + ks * 32);
      // home: four stages in the 256 accumulation registers (MFMA operands read
      // them there), the fifth in vector registers
      if (i < 4) asm volatile("" : "+a"(Wr[i][ks]));
      else asm volatile("" : "+v"(Wr[i][ks]));
    }
  }

  // backbone rows of slot group g: 16-byte chunk p of the buffer (p = 64 j +
  // lane for instruction j) is chunk c = p mod rs of row p / rs; padding chunks
  // and rows past the batch load a valid chunk that is never read; chunks past
  // V (in the last tile) load kNegInfChunk.
  // Addresses are a uniform base (the group's first row) plus a 32-bit lane
  // offset (the launcher checks that 32 rows fit).
  auto dma_x = [&](int pos, int g) {
    const char* gbase = Xb + ((size_t)g * 32 * gamma + pos) * (size_t)V * 2;
    const uint32_t rows = (uint32_t)min(32, B - g * 32), rowb = (uint32_t)gamma * (uint32_t)V * 2u;
    uint32_t ln = (uint32_t)lane;
    asm volatile("" : "+v"(ln));  // computed here, not kept live across the loop
#pragma unroll
    for (int m = 0; m < kResXInstr; ++m) {
      const uint32_t j = (uint32_t)(wave * kResXInstr + m);
      const uint32_t p = j * 64u + ln;
      uint32_t row = __umulhi(p, rs_magic);
      uint32_t c = p - row * rs;
      if (row >= rows || c >= nch) row = 0, c = 0;
      const uint32_t col = (uint32_t)T0 * 64u + c * 8u;
      const void* src = col < (uint32_t)V ? static_cast<const void*>(gbase + (row * rowb + col * 2u))
                                          : static_cast<const void*>(&kNegInfChunk);
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(lds + (g & 1) * kResXBufBytes + j * 1024), 16, 0, 0);
    }
  };
  // U rows of slot group g: chunk c of slot s at 16-byte position 32 s + (c ^ s),
  // so that the B-operand reads of 16 consecutive slots hit distinct banks
  auto dma_u = [&](int g) {
    int hv = half;
    asm volatile("" : "+v"(hv));  // computed here, not kept live across the loop
#pragma unroll
    for (int m = 0; m < U_DMA; ++m) {
      const int j = wave * U_DMA + m;
      const int s = 2 * j + hv;
      const uint32_t tk = (uint32_t)gs.tok[min(g * 32 + s, B - 1)];
      __builtin_amdgcn_global_load_lds(Ub + (tk * (uint32_t)(R * 2) + (uint32_t)((l32 ^ s) * 16)),
                                       (lds_ptr_t)(reinterpret_cast<char*>(gs.urows[g & 1]) + j * 1024), 16, 0, 0);
    }
  };

  // the tile records of slot group g: merge the two stages of each tile.  The
  // stores (write-through, slow to complete) count in vmcnt with the direct
  // loads, so they are issued one group after the statistics, right after a
  // group's wait: they then have a group's work to complete before the next
  // wait, which could otherwise only pass after loads issued just before it.
  auto records = [&](int g) {
    for (int q = tid; q < 32 * ntl; q += 256) {
      const int sl = q / ntl, t = q - sl * ntl;
      const int b = g * 32 + sl;
      if (b < B) {
        float2 f, s2;
        float c;
        lds_load_record_parts(&gs.st[g & 1][2 * t][sl], &gs.st[g & 1][2 * t + 1][sl], &cTs[b], f, s2, c);
        const float m = fmaxf(f.x, s2.x);
        float s = f.y * __builtin_amdgcn_exp2f((f.x - m) * c);
        if (s2.y > 0.0f) s += s2.y * __builtin_amdgcn_exp2f((s2.x - m) * c);
        store_rec_coherent(static_cast<TileStat*>(const_cast<void*>(a.tstat)) + (size_t)b * nt + T0 + t, m, s);
      }
    }
  };

  uint32_t phase = 0;
  for (int pos = 0; pos < gamma; ++pos) {
    // previous tokens: prev0 at position 0, else the draws of this launch
    // (clamped into [0, V): a draw that never ran, after a stalled wait, leaves
    // whatever the output held)
    for (int b = tid; b < B; b += 256)
      gs.tok[b] = pos == 0 ? checked_token(a.prev0[b], V, a.status, kBadPrev)
                           : min(max(load_coherent(a.draft + (size_t)b * gamma + pos - 1), 0), V - 1);
    __syncthreads();
    dma_x(pos, 0);
    if (NG > 1) dma_x(pos, 1);
    dma_u(0);
    if (NG > 1) dma_u(1);

    for (int g = 0; g < NG; ++g) {
      // group g's loads have landed in every wavefront (the next group's may be
      // in flight; record stores are counted too, which only waits longer)
      if (g + 1 >= NG) wait_vmcnt_c<0>();
      else if (g == 0) wait_vmcnt_c<U_DMA>();
      else wait_vmcnt_c<X_DMA + U_DMA>();
      barrier_only();
      if (g > 0) records(g - 1);

      bf16x8 H[KS];
      {
        // chunk 2 ks + half of slot l32: byte (32 ks) ^ sw past the slot's row
        uint32_t sw = (uint32_t)(half ^ l32) * 16u;
        asm volatile("" : "+v"(sw));  // computed here, not kept live across the loop
        const char* ub = reinterpret_cast<const char*>(gs.urows[g & 1]) + l32 * 512;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          H[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ub + ((uint32_t)(32 * ks) ^ sw)));
      }
      const float cT = cTs[min(g * 32 + l32, B - 1)];
      const char* const xrow = lds + (g & 1) * kResXBufBytes + (uint32_t)l32 * rs * 16u;  // this lane's slot
      // Stage i's statistics run interleaved with the MFMAs of stage i + 1
      // (one wavefront per SIMD: the matrix core works while the vector unit
      // forms t, its maximum and its exp2-sum): per k-step, the first quarter
      // forms t = x + bias for 4 columns, the second takes their
      // maximum, the second half adds 2 exp2 terms.
      const f32x16 zero = {};
      f32x16 acc[2];
      acc[0] = zero;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Wr[0][ks], H[ks], acc[0], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        f32x16& cur = acc[i & 1];
        f32x16& nxt = acc[(i + 1) & 1];
        const int cs = S0 + i;  // stage index within the workgroup
        // columns 16 half .. + 15 of the stage
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(xrow + (cs * 4 + 2 * half) * 16);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(xrow + (cs * 4 + 2 * half) * 16 + 16);
        float tmax = -INFINITY, sum = 0.0f, mc = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (i + 1 < KW)
            nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Wr[i + 1 < KW ? i + 1 : i][ks], H[ks], ks == 0 ? zero : nxt,
                                                          0, 0, 0);
          if (ks < 4) {
#pragma unroll
            for (int e = 4 * ks; e < 4 * ks + 4; ++e) {
              const uint32_t w = e < 8 ? w0[(e & 7) >> 1] : w1[(e & 7) >> 1];
              const float x = (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
              cur[e] = x + cur[e];  // columns past V: x = -inf
            }
          } else if (ks < 8) {
#pragma unroll
            for (int e = 4 * (ks - 4); e < 4 * (ks - 4) + 4; ++e) tmax = fmaxf(tmax, cur[e]);
            if (ks == 7) tmax = pair_max(tmax), mc = tmax * cT;
          } else {
#pragma unroll
            for (int e = 2 * (ks - 8); e < 2 * (ks - 8) + 2; ++e) sum += __builtin_amdgcn_exp2f(fmaf(cur[e], cT, -mc));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        sum = pair_sum(sum);
        const bool mine = i < nsw;
        if (half == 0) {
          // LDS that no direct load targets: written without the compiler's wait
          // for the direct loads in flight (the waits before the barrier cover it)
          lds_store_f32x2(&gs.st[g & 1][mine ? cs : kResWaves * KW][l32], tmax, sum);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_only();  // statistics complete; ring slot g & 1 and U rows g & 1 free again
      // (stage statistics of g stay until the records of g are made at the top of
      // group g + 1: group g + 2, the next to write them, starts after that)
      if (g + 2 < NG) {
        dma_x(pos, g + 2);
        dma_u(g + 2);
      }
    }
    records(NG - 1);

    // every record of this position is written: draw
    wait_vmcnt_c<0>();
    grid_phase(ra, ++phase);
    DraftSelectArgs d = a;
    d.pos = pos;
    for (int b = cu; b < B; b += G) {
      draft_select_block<uint16_t, uint16_t, true>(d, b, dsh);
      __syncthreads();
    }
    if (pos + 1 < gamma) {
      wait_vmcnt_c<0>();
      grid_phase(ra, ++phase);
    }
  }

  // the last workgroup out leaves the flags at zero
  wait_vmcnt_c<0>();
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(ra.exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (uint32_t)G - 1) {
      for (int i = 0; i < G; ++i) __hip_atomic_store(ra.flags + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ra.exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
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
  // Walker w = blockIdx.x - group walkers runs on XCD w % 8 and takes tiles
  // run_pos, run_pos + walkers, ...: in each round of `walkers` tiles, the
  // walkers of one XCD take walkers / 8 adjacent tiles, so the 4-byte masses
  // of neighbouring tiles of a slot's row meet in one L2 and leave it as whole
  // lines (dealt round robin, each line was written back piecemeal by 8 L2s).
  const int w = (int)blockIdx.x - group * walkers;
  const int run_pos = (walkers & 7) == 0 ? (w & 7) * (walkers >> 3) + (w >> 3) : w;
  if (group >= ngroups || run_pos >= nt) return;  // uniform
  const int sg0 = group * kResSlots;
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);

  int rq, pos, prev;
  bool valid;
  slot_info<true>(a, sg0 + sl, nslots, rq, pos, prev, valid);
  const bool active = sg0 + (wave & 3) * 32 < nslots;
  // p = 2^((z - max) c - ln S log2 e): the difference first (max is an exact
  // input value), so no term carries an error proportional to max / T
  float T = 1.0f, mz = 0.0f, kp = 0.0f;
  double lse_q = 0.0;
  if (valid) {
    T = effective_temp(a.temperature[rq]);
    const ReqState st = a.req[rq];
    mz = (float)st.row_max;
    kp = (float)(st.row_logsum * 1.4426950408889634);
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
      const float p = __builtin_amdgcn_exp2f(fmaf(zv[e] - mz, c, -kp));
      const float q = __builtin_amdgcn_exp2f(fmaf((xv[e] - ref) + acc[e], c, -kq));
      rs += fmaxf(p - q, 0.0f);
    }
    return reduce_pair32(rs, OpSum{});
  };

  const int G = walkers;
  int t = run_pos;
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

// ---------------------------------------------------------------------------
// Streaming residual-mode pass (bf16 logits with V a multiple of 8, bf16
// factors, R in {128, 256}): the draft kernel's design with a third stream.
// A workgroup of 8 wavefronts owns 256 slots and walks 64-column tiles as two
// 32-column stages; W2 rows (shared) and each wavefront's backbone and target
// rows (private) reach LDS by direct loads into three-stage rings, two stages
// ahead.  Iteration u issues the MFMAs of stage u+1 (the accumulator sums the
// bias alone; t = (x - ref) + bias is formed with one rounding) with the
// masses of stage u: per
// column p = exp(z / T - ln Z_p), q = exp((ref + t) / T - lse_q) and
// max(0, p - q) (the residual draw) or min(p, q) (the acceptance pass).  The
// residual draw needs each tile's mass; the acceptance pass only the total, so
// a slot's masses are summed in fp64 across the workgroup's tiles and written
// once per workgroup (column blockIdx.x of the slot's row of partial sums).
// ---------------------------------------------------------------------------
constexpr int kRStages = 3;

template <int R, bool TV>
__global__ __launch_bounds__(512, 1) void gemm_residual_stream(GemmArgs a) {
  using WL = WLayout<R, kStageCols>;
  constexpr int KS = R / 16;
  constexpr int W_DMA = WL::NB / 8;
  constexpr int X_DMA = kXStageBytes / 1024;
  constexpr int W_RING = kRStages * WL::BYTES;
  constexpr int SLOT_BYTES = 2 * kXStageBytes;  // backbone then target logits of one stage
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nslots = residual_slots(a);
  const int sg0 = blockIdx.y * kSlotsPerGroup;
  const int nt = a.n_tiles, G = gridDim.x;
  if (sg0 >= nslots || (int)blockIdx.x >= nt) return;  // uniform across the workgroup
  const int V = a.V;
  char* const ring = lds + W_RING + wave * (kRStages * SLOT_BYTES);  // this wave's logit ring
  const char* const Wb = static_cast<const char*>(a.Wt);
  const char* const Xb = static_cast<const char*>(a.base);
  const char* const Zb = static_cast<const char*>(a.target);

  const int n_stage = 2 * ((nt - 1 - (int)blockIdx.x) / G + 1);
  auto stage_col = [&](int u) {
    u = min(u, n_stage - 1);
    return ((int)blockIdx.x + (u >> 1) * G) * kTile + (u & 1) * kStageCols;
  };
  auto dma_w = [&](int u, int slot) {
    const int c0 = stage_col(u);
#pragma unroll
    for (int k = 0; k < W_DMA; ++k) {
      const int f = wave + 8 * k;
      const int s = f * WL::RB + lane % WL::RB, c = lane / WL::RB;
      const int v = min(c0 + col_of_row(s), V - 1);
      __builtin_amdgcn_global_load_lds(Wb + ((uint32_t)v * (R * 2) + c * 16),
                                       (lds_ptr_t)(lds + slot * WL::BYTES + WL::block(f)), 16, 0, 0);
    }
  };

  // this wave's 32 slots (compiler-visible loads, all waited for before the
  // first stream load is issued)
  int rq, pos, prev;
  bool valid;
  slot_info<true>(a, sg0 + wave * 32 + l32, nslots, rq, pos, prev, valid);
  float T = valid ? effective_temp(a.temperature[rq]) : 1.0f;
  if (!(T > 0.0f)) T = 1.0f;  // greedy rows: no residual draw; the acceptance pass ignores their masses
  double rmax = 0.0, rlsum = 0.0, lse_q = 0.0;
  if (valid) {
    residual_rowstats(a, rq, pos, rmax, rlsum);
    lse_q = a.draft_lse[(size_t)rq * a.gamma + pos];
  }
  bf16x8 H[KS];
  {
    const uint16_t* h = static_cast<const uint16_t*>(a.U) + (size_t)prev * R + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) H[ks] = *reinterpret_cast<const bf16x8*>(h + ks * 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0070 | (0xF << 8));  // vmcnt(0)
  const double invT = 1.0 / (double)T;
  const float cT = kLog2e / T;
  // p = 2^((z - max) c - ln S log2 e): the difference first (max is an exact
  // input value), so no term carries an error proportional to max / T
  const float mz = (float)rmax, kp = (float)(rlsum * 1.4426950408889634);
  asm volatile("" : "+v"(lse_q));  // every register load is consumed here, before the streams start
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t xrow = (uint32_t)(rq * a.gamma + pos) * (uint32_t)V;
  const uint32_t zrow = (uint32_t)(rq * (a.gamma + 1) + pos) * (uint32_t)V;
  // lane L of direct load k fetches chunk 2k + L / 32 of slot L % 32's row
  auto dma_xz = [&](int u, int slot) {
    const int c0 = stage_col(u);
#pragma unroll
    for (int k = 0; k < X_DMA; ++k) {
      const int col = min(c0 + (2 * k + half) * 8, V - 8);
      __builtin_amdgcn_global_load_lds(Xb + (xrow + (uint32_t)col) * 2u,
                                       (lds_ptr_t)(ring + slot * SLOT_BYTES + k * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < X_DMA; ++k) {
      const int col = min(c0 + (2 * k + half) * 8, V - 8);
      __builtin_amdgcn_global_load_lds(Zb + (zrow + (uint32_t)col) * 2u,
                                       (lds_ptr_t)(ring + slot * SLOT_BYTES + kXStageBytes + k * 1024), 16, 0, 0);
    }
  };
  constexpr int STAGE_LOADS = W_DMA + 2 * X_DMA;
  dma_w(0, 0);
  dma_xz(0, 0);
  dma_w(1, 1);
  dma_xz(1, 1);
  dma_w(2, 2);
  dma_xz(2, 2);

  const int wbase = WL::at(l32, half);
  const int xbase = half * 1024 + l32 * 16;
  auto read16 = [&](int slot, int off, u32x4& w0, u32x4& w1) {
    w0 = *reinterpret_cast<const u32x4*>(ring + slot * SLOT_BYTES + off + xbase);
    w1 = *reinterpret_cast<const u32x4*>(ring + slot * SLOT_BYTES + off + xbase + 512);
  };
  auto unpack = [](const u32x4& w0, const u32x4& w1, int e) {
    const uint32_t w = e < 8 ? w0[(e & 7) >> 1] : w1[(e & 7) >> 1];
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  };
  // the accumulator starts at zero (the bias alone, at its own scale); the
  // first stage of a tile sets ref
  auto seed = [&](int slot, bool first, f32x16& acc, float& ref) {
    if (first) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(ring + slot * SLOT_BYTES + xbase);
      float even, odd;
      row_pair<32>(__uint_as_float(w << 16), even, odd);
      ref = even;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  };
  auto rd = [&](int slot, int ks) {
    return *reinterpret_cast<const bf16x8*>(lds + slot * WL::BYTES + wbase + 32 * WL::RB * ks);
  };
  // MFMAs of the next stage interleaved with the masses of the current one
  auto fused = [&](int slot, const f32x16& cur, const float (&z)[16], float kq, f32x16& next) {
    float m = 0.0f;
    bf16x8 A[2];
    A[0] = rd(slot, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) A[(ks + 1) & 1] = rd(slot, ks + 1);
      next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks & 1], H[ks], next, 0, 0, 0);
      constexpr int n = 16 / KS > 0 ? 16 / KS : 1;  // columns of the current stage per k-step
      if (ks * n < 16) {
#pragma unroll
        for (int j = ks * n; j < ks * n + n; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(z[j] - mz, cT, -kp));
          const float q = __builtin_amdgcn_exp2f(fmaf(cur[j], cT, -kq));
          m += TV ? fminf(p, q) : fmaxf(p - q, 0.0f);
        }
        asm volatile("" : "+v"(m));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return pair_sum(m);
  };

  f32x16 acc0, acc1;
  float ref0 = 0.0f, ref1 = 0.0f, tile_mass = 0.0f;
  double total = 0.0;  // acceptance pass: this slot's masses over the workgroup's tiles
  int tile = blockIdx.x;
  wait_vmcnt_c<2 * STAGE_LOADS>();  // stage 0 landed
  barrier_only();
  seed(0, true, acc0, ref0);
  ref1 = ref0;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd(0, ks), H[ks], acc0, 0, 0, 0);
  wait_vmcnt_c<STAGE_LOADS>();  // stage 1 landed
  barrier_only();

  // Iteration u (stage u in ring slot S = u % 3, its bias in `cur`):
  //   take stage u's backbone and target logits into registers, seed `next`,
  //   issue stage u+3 into slot S, run stage u+1's
  //   MFMAs with stage u's masses, on a tile's second stage store the tile's
  //   mass (residual draw), wait for stage u+2 (issued in iteration u-1, or
  //   the prologue), barrier.
  auto step = [&](auto S_, auto second_, f32x16& cur, f32x16& next, int u) {
    constexpr int S = decltype(S_)::value;
    constexpr bool second = decltype(second_)::value;
    u32x4 xw0, xw1, zw0, zw1;
    read16(S, 0, xw0, xw1);
    read16(S, kXStageBytes, zw0, zw1);
    seed((S + 1) % kRStages, second, next, ref0);
    float z[16], x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = unpack(zw0, zw1, e), x[e] = unpack(xw0, xw1, e);
    // slot S is rewritten below: its logits must have reached registers
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_w(u + 3, S);
    dma_xz(u + 3, S);
#pragma unroll
    for (int e = 0; e < 16; ++e) cur[e] = (x[e] - ref1) + cur[e];  // t = (x - ref) + bias, one rounding
    const int c0 = tile * kTile + (second ? kStageCols : 0);
    if (c0 + kStageCols > V) {  // a ragged stage: columns >= V do not exist
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (c0 + half * 16 + e >= V) cur[e] = -INFINITY, z[e] = -INFINITY;
    }
    const float kq = (float)((lse_q - (double)ref1 * invT) * 1.4426950408889634);
    const float m = fused((S + 1) % kRStages, cur, z, kq, next);
    tile_mass += m;
    if (second) {
      if (TV) total += (double)tile_mass;
      else if (half == 0 && valid) a.rsum[residual_out(a, rq, pos, tile)] = tile_mass;
      tile_mass = 0.0f;
      tile += G;
      ref1 = ref0;
    }
    wait_vmcnt_c<STAGE_LOADS>();
    barrier_only();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using F = std::false_type;
  using Tt = std::true_type;
  for (int u = 0;; u += 6) {
    step(I0{}, F{}, acc0, acc1, u + 0); if (u + 1 >= n_stage) break;
    step(I1{}, Tt{}, acc1, acc0, u + 1); if (u + 2 >= n_stage) break;
    step(I2{}, F{}, acc0, acc1, u + 2); if (u + 3 >= n_stage) break;
    step(I0{}, Tt{}, acc1, acc0, u + 3); if (u + 4 >= n_stage) break;
    step(I1{}, F{}, acc0, acc1, u + 4); if (u + 5 >= n_stage) break;
    step(I2{}, Tt{}, acc1, acc0, u + 5); if (u + 6 >= n_stage) break;
  }
  if (TV && half == 0 && valid)
    a.rsum[((size_t)rq * a.gamma + pos) * a.n_tiles + blockIdx.x] = (float)total;
}

template <int R>
hipError_t launch_residual_stream(const GemmArgs& a, hipStream_t s, int* parts) {
  const size_t lds = (size_t)kRStages * (WLayout<R, kStageCols>::BYTES + 8 * 2 * kXStageBytes);
  const void* fn = a.tv ? reinterpret_cast<const void*>(&gemm_residual_stream<R, true>)
                       : reinterpret_cast<const void*>(&gemm_residual_stream<R, false>);
  int mw = 0;
  const hipError_t e = kernel_setup(fn, 512, lds, &mw);
  if (e != hipSuccess) return e;
  // the residual draw may need every request; the acceptance pass has B gamma slots
  const int groups = (max_slots(a, true) + kSlotsPerGroup - 1) / kSlotsPerGroup;
  const int wg_x = max(1, min(a.n_tiles, mw / groups));
  if (parts) *parts = wg_x;
  if (a.tv) launch(&gemm_residual_stream<R, true>, dim3(wg_x, groups), 512, lds, s, a);
  else launch(&gemm_residual_stream<R, false>, dim3(wg_x, groups), 512, lds, s, a);
  return hipGetLastError();
}

template <int R>
hipError_t launch_residual_coalesced(const GemmArgs& a, hipStream_t s) {
  const size_t lds = (size_t)2 * (kTile * R * 2) + (size_t)4 * (kResSlots * kTile * 2);
  int max_wg = 0;
  const hipError_t e = kernel_setup(reinterpret_cast<const void*>(&gemm_residual_coalesced<R>), 512, lds, &max_wg);
  if (e != hipSuccess) return e;
  // enough workgroups to give every CU one, and at least one per tile of every
  // possible slot group when the batch is small
  const int groups = (max_slots(a, true) + kResSlots - 1) / kResSlots;
  const int grid = max(8, min(max_wg, groups * a.n_tiles));
  launch(&gemm_residual_coalesced<R>, grid, 512, lds, s, a);
  return hipGetLastError();
}

template <typename TL, bool RESIDUAL, int R>
hipError_t launch_pipelined(const GemmArgs& a, hipStream_t s) {
  const size_t lds = (size_t)kRing * (2 * (R / 16) * 1024);
  int max_wg = 0;
  const hipError_t e =
      kernel_setup(reinterpret_cast<const void*>(&gemm_stats_lds<TL, RESIDUAL, R>), 64 * kLdsWaves, lds, &max_wg);
  if (e != hipSuccess) return e;
  const int groups = (max_slots(a, RESIDUAL) + kSlotsPerGroup - 1) / kSlotsPerGroup;
  const int threads = 64 * min(kLdsWaves, (max_slots(a, RESIDUAL) + 31) / 32);
  const int wg_x = max(1, min(a.n_tiles, max_wg / groups));
  launch(&gemm_stats_lds<TL, RESIDUAL, R>, dim3(wg_x, groups), threads, lds, s, a);
  return hipGetLastError();
}

template <typename TL, bool RESIDUAL>
hipError_t gemm_dispatch(const GemmArgs& a, int factor_dtype, bool vec, hipStream_t s, int* parts) {
  if (parts) *parts = a.n_tiles;  // one partial per tile unless the streaming pass says otherwise
  if constexpr (sizeof(TL) == 2) {
    // the coalesced kernels address their inputs with 32-bit byte offsets
    const bool fits = (size_t)a.B * (a.gamma + 1) * a.V * 2 < (1ull << 32) &&
                      (size_t)a.V * a.r * 2 < (1ull << 32) && (size_t)(a.B + 1) * a.n_tiles * 16 < (1ull << 32);
    if (factor_dtype == DSPARK_BF16 && a.V % 8 == 0 && a.V >= 64 && (a.r == 128 || a.r == 256) && fits) {
      if constexpr (RESIDUAL) {
        // the residual draw (at most B rows): the coalesced kernel; the acceptance
        // pass (B gamma rows): the streaming one
        if (!a.tv) return a.r == 256 ? launch_residual_coalesced<256>(a, s) : launch_residual_coalesced<128>(a, s);
        if (a.r == 256) return launch_residual_stream<256>(a, s, parts);
        return launch_residual_stream<128>(a, s, parts);
      } else {
        if (a.r == 256) return launch_draft_stream<256>(a, s);
        return launch_draft_stream<128>(a, s);
      }
    }
  }
  if (factor_dtype == DSPARK_BF16 && vec && (a.r == 64 || a.r == 128 || a.r == 256)) {
    if (a.r == 256) return launch_pipelined<TL, RESIDUAL, 256>(a, s);
    if (a.r == 128) return launch_pipelined<TL, RESIDUAL, 128>(a, s);
    return launch_pipelined<TL, RESIDUAL, 64>(a, s);
  }
  if (factor_dtype == DSPARK_BF16 && a.r % 16 == 0) {
    const dim3 grid(a.n_tiles, (max_slots(a, RESIDUAL) + 255) / 256);
    if (vec) launch(&gemm_stats_mfma<TL, RESIDUAL, true>, grid, 256, 0, s, a);
    else launch(&gemm_stats_mfma<TL, RESIDUAL, false>, grid, 256, 0, s, a);
  } else {
    const dim3 grid(a.n_tiles, max_slots(a, RESIDUAL));
    if (factor_dtype == DSPARK_BF16) launch(&gemm_stats_valu<TL, uint16_t, RESIDUAL>, grid, 64, 0, s, a);
    else launch(&gemm_stats_valu<TL, float, RESIDUAL>, grid, 64, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_stats(const GemmArgs& a, int logits_dtype, int factor_dtype, bool residual,
                             hipStream_t s, int* parts) {
  const bool vec = a.V % 4 == 0;
  if (logits_dtype == DSPARK_BF16)
    return residual ? gemm_dispatch<uint16_t, true>(a, factor_dtype, vec, s, parts)
                    : gemm_dispatch<uint16_t, false>(a, factor_dtype, vec, s, parts);
  return residual ? gemm_dispatch<float, true>(a, factor_dtype, vec, s, parts)
                  : gemm_dispatch<float, false>(a, factor_dtype, vec, s, parts);
}

template <typename TL, typename TF>
hipError_t launch_select_schedule_t(const DraftSelectArgs& d, const ScheduleArgs& sa, hipStream_t stream) {
  // the scheduler's dynamic LDS reaches 80 KB at B gamma = 8192 with a 1024-point table
  int unused = 0;
  const hipError_t e = kernel_setup(reinterpret_cast<const void*>(&draft_select_schedule<TL, TF>), 256,
                                    8192 * 8 + 1024 * 16, &unused);
  if (e != hipSuccess) return e;
  const SelectScheduleArgs a{d, sa};
  launch(&draft_select_schedule<TL, TF>, dim3(d.B + schedule_groups(sa)), 256, schedule_lds_bytes(sa), stream, a);
  return hipGetLastError();
}

hipError_t launch_draft_select_schedule(const DraftSelectArgs& d, const ScheduleArgs& sa, int logits_dtype,
                                        int factor_dtype, hipStream_t stream) {
  if (d.n_tiles > kTilesPerBlock * 64) return hipErrorNotSupported;
  if (logits_dtype == DSPARK_BF16)
    return factor_dtype == DSPARK_BF16 ? launch_select_schedule_t<uint16_t, uint16_t>(d, sa, stream)
                                       : launch_select_schedule_t<uint16_t, float>(d, sa, stream);
  return factor_dtype == DSPARK_BF16 ? launch_select_schedule_t<float, uint16_t>(d, sa, stream)
                                     : launch_select_schedule_t<float, float>(d, sa, stream);
}

// Bound of the resident round's device-wide waits, in s_memrealtime ticks
// (100 MHz); 0.2 s unless set.
static std::atomic<uint64_t> g_resident_wait_ticks{20000000ull};

uint64_t set_resident_wait_ticks(uint64_t ticks) { return g_resident_wait_ticks.exchange(ticks); }

hipError_t launch_draft_resident(const DraftSelectArgs& d, int logits_dtype, int factor_dtype,
                                 uint32_t* grid_words, hipStream_t s) {
  static_assert(kResMaxGrid + 1 <= kResidentGridWords, "phase flags and exit counter");
  // lane offsets within a slot group's 32 rows and within U are 32-bit
  const bool fits = (size_t)32 * d.gamma * d.V * 2 < (1ull << 32) && (size_t)d.V * d.r * 2 < (1ull << 32);
  if (logits_dtype != DSPARK_BF16 || factor_dtype != DSPARK_BF16 || d.r != 256 || d.V % 8 != 0 || d.V < 64 ||
      d.B > kResMaxB || d.n_tiles > kDrawMaxTiles || d.hrows || !fits)
    return hipErrorNotSupported;
  int dev = 0, cus = 0, coop = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (e != hipSuccess) return e;
  // W2 must fit: at most 2 kResStagesPerWave tiles per workgroup
  if (!coop || cus < 1 || cus > kResMaxGrid || (d.n_tiles + cus - 1) / cus > 2 * kResStagesPerWave)
    return hipErrorNotSupported;
  int groups = 0;
  e = kernel_setup(reinterpret_cast<const void*>(&draft_round_resident), 256, kResLdsBytes, &groups);
  if (e != hipSuccess) return e;
  if (groups < cus) return hipErrorNotSupported;
  ResidentArgs ra{};
  ra.d = d;
  ra.flags = grid_words;
  ra.exits = grid_words + kResMaxGrid;
  ra.spin_limit = g_resident_wait_ticks.load(std::memory_order_relaxed);
  void* args[] = {&ra};
  KernelEvents* ev = kernel_events();
  if (ev && ev->launches == 0) (void)hipEventRecord(ev->start, s);
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&draft_round_resident), dim3(cus), dim3(256), args,
                                 (unsigned)kResLdsBytes, s);
  if (e != hipSuccess) {
    // Nothing was enqueued.  The runtime refuses a cooperative launch with
    // hipErrorIllegalState while another process on the device holds its
    // cooperative-launch resources: the caller then takes the per-position
    // launches, with the error cleared so that their checks do not report it.
    (void)hipGetLastError();
    return e == hipErrorIllegalState || e == hipErrorCooperativeLaunchTooLarge ? hipErrorNotSupported : e;
  }
  if (ev && hipEventRecord(ev->stop, s) == hipSuccess) ++ev->launches;
  return hipSuccess;
}

hipError_t launch_draft_select(const DraftSelectArgs& a, int logits_dtype, int factor_dtype,
                               hipStream_t s) {
  const dim3 grid(a.B);
  if (a.n_tiles <= kTilesPerBlock * 64) {
    if (logits_dtype == DSPARK_BF16) {
      if (factor_dtype == DSPARK_BF16) launch(&draft_select_fast<uint16_t, uint16_t>, grid, 512, 0, s, a);
      else launch(&draft_select_fast<uint16_t, float>, grid, 512, 0, s, a);
    } else {
      if (factor_dtype == DSPARK_BF16) launch(&draft_select_fast<float, uint16_t>, grid, 512, 0, s, a);
      else launch(&draft_select_fast<float, float>, grid, 512, 0, s, a);
    }
    return hipGetLastError();
  }
  if (logits_dtype == DSPARK_BF16) {
    if (factor_dtype == DSPARK_BF16) launch(&draft_select_kernel<uint16_t, uint16_t>, grid, 256, 0, s, a);
    else launch(&draft_select_kernel<uint16_t, float>, grid, 256, 0, s, a);
  } else {
    if (factor_dtype == DSPARK_BF16) launch(&draft_select_kernel<float, uint16_t>, grid, 256, 0, s, a);
    else launch(&draft_select_kernel<float, float>, grid, 256, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark

// Device-side building blocks of the DSpark round for gfx950: the counter-based
// generator, bf16 handling, 64-lane wavefront reductions and the record types
// kernels exchange through the workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

// Sampler partition: 64 elements per tile, 64 tiles per block.
constexpr int kTile = 64;
constexpr int kTilesPerBlock = 64;
constexpr int kBlock = kTile * kTilesPerBlock;

// Philox streams: which decision of the round a draw feeds.
enum : uint32_t {
  kDraftTop = 0, kDraftMid = 1, kDraftLeaf = 2,
  kAccept = 3,
  kFinalTop = 4, kFinalMid = 5, kFinalLeaf = 6,
};

// Bits of the workspace status word.  kStall: a device-wide wait of the
// resident draft round passed its time bound (its results are then unspecified).
enum : uint32_t {
  kBadPrev = 1u, kBadDraft = 2u, kBadBudget = 4u, kBadTemp = 8u, kBadConf = 16u, kBadTable = 32u,
  kStall = 64u,
};

// Softmax statistics of one 64-column tile of one draft row, d(v) being the
// draft logit (backbone logit x(v) plus Markov bias) and T the temperature.
// bf16 logits: t(v) = x(v) + bias(v) with one rounding (x is exact in fp32),
//   mx = max_v t(v), sum = sum_v exp((t(v) - mx) / T); d(v) = t(v).
struct TileStat {
  float mx, sum;
};
// fp32 logits: the same with t(v) = (x(v) - ref) + bias(v), ref the tile's
// largest backbone logit, so that the terms near the maximum carry no rounding
// proportional to |ref| / T; d(v) = ref + t(v).
struct TileStatRef {
  float ref, mx, sum, pad;
};
template <typename TL> struct TileRecOf { using type = TileStatRef; };
template <> struct TileRecOf<uint16_t> { using type = TileStat; };
template <typename TL> using TileRec = typename TileRecOf<TL>::type;
// the tile's largest draft logit (exact: a sum of two fp32 values in fp64)
__device__ __forceinline__ double rec_top(const TileStat& r) { return (double)r.mx; }
__device__ __forceinline__ double rec_top(const TileStatRef& r) { return (double)r.ref + (double)r.mx; }

// Statistics of one 4096-column block of one target row:
//   mx = max z (an input value), sum = sum exp((z - mx) / T), arg = lowest index
//   of mx (greedy requests only).
struct BlockStat {
  float mx, sum;
  int arg;
  float pad;
};

// Per-request state handed from the accept pass to the residual pass.
struct ReqState {
  double row_max;    // max of target row n (an input value)
  double row_logsum; // ln sum exp((z - row_max) / T) over target row n
  double res_mass;   // total residual mass of the row (set by the residual draw)
  int n;             // accepted count
  int pending;       // the final token still to be drawn: kDrawResidual or kDrawBonus, else 0
};
enum : int { kDrawResidual = 1, kDrawBonus = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

template <typename TL> __device__ __forceinline__ float load_logit(const TL* p);
template <> __device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}
template <> __device__ __forceinline__ float load_logit<float>(const float* p) { return *p; }

// ---------------------------------------------------------------------------
// Philox4x32-10 (J. K. Salmon et al., "Parallel Random Numbers: As Easy as 1,
// 2, 3", SC'11): per round, words 0 and 2 are multiplied by two odd constants;
// the high halves are xored with words 1 and 3 and the round key, the low
// halves become the new words 1 and 3.  The key advances by two Weyl
// increments between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Draw n of (stream, request, position): word n % 4 of the block n / 4.
__device__ __forceinline__ uint32_t rng_word(uint64_t seed, uint32_t stream, uint32_t req,
                                             uint32_t pos, uint32_t n) {
  const uint4 o = philox4x32_10(make_uint4(n >> 2, pos, req, stream), (uint32_t)seed,
                                (uint32_t)(seed >> 32));
  const uint32_t j = n & 3u;
  return j == 0 ? o.x : j == 1 ? o.y : j == 2 ? o.z : o.w;
}

// Uniform in (0, 1): the odd multiples of 2^-24, from the top 23 bits.
__device__ __forceinline__ double uniform_from_word(uint32_t w) {
  return ((double)(w >> 9) + 0.5) * 0x1p-23;
}

__device__ __forceinline__ double gumbel_from_word(uint32_t w) {
  return -log(-log(uniform_from_word(w)));
}

__device__ __forceinline__ double gumbel(uint64_t seed, uint32_t stream, uint32_t req, uint32_t pos,
                                         uint32_t n) {
  return gumbel_from_word(rng_word(seed, stream, req, pos, n));
}

// ---------------------------------------------------------------------------
// Lane exchanges without LDS.  Inside a row of 16 lanes: DPP quad permutes
// (lane ^ 1, lane ^ 2) and the mirrors (lane i <-> 7 - i within 8, 15 - i within
// 16).  Across rows: gfx950's v_permlane16_swap / v_permlane32_swap; swapping a
// register with itself returns, in both results, the even and the odd row (row
// pair) of each pair, so op(first, second) is the pairwise result.  Each step of
// a reduction combines two values that are identical in the two lanes it joins,
// so every lane ends with the bitwise same result; a 16-lane reduction is four
// dependent VALU moves, a 64-lane one six.
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <typename T> __device__ __forceinline__ uint64_t to_bits(T v) {
  if constexpr (sizeof(T) == 8) return __builtin_bit_cast(uint64_t, v);
  else return (uint64_t)__builtin_bit_cast(uint32_t, v);
}
template <typename T> __device__ __forceinline__ T from_bits(uint64_t b) {
  if constexpr (sizeof(T) == 8) return __builtin_bit_cast(T, b);
  else return __builtin_bit_cast(T, (uint32_t)b);
}
template <int CTRL, typename T> __device__ __forceinline__ T dpp(T v) {
  const uint64_t b = to_bits(v);
  uint64_t r = dpp_u32<CTRL>((uint32_t)b);
  if constexpr (sizeof(T) == 8) r |= (uint64_t)dpp_u32<CTRL>((uint32_t)(b >> 32)) << 32;
  return from_bits<T>(r);
}
// (value of the even row of the pair, value of the odd row), rows of 16 (W = 16)
// or halves of 32 (W = 32)
template <int W, typename T> __device__ __forceinline__ void row_pair(T v, T& even, T& odd) {
  const uint64_t b = to_bits(v);
  uint64_t e, o;
  {
    const auto r = W == 16 ? __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false)
                           : __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    e = r[0], o = r[1];
  }
  if constexpr (sizeof(T) == 8) {
    const uint32_t hi = (uint32_t)(b >> 32);
    const auto r = W == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                           : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    e |= (uint64_t)r[0] << 32, o |= (uint64_t)r[1] << 32;
  }
  even = from_bits<T>(e), odd = from_bits<T>(o);
}

template <typename T, typename Op> __device__ __forceinline__ T reduce16(T v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppMirror>(v));
  return v;
}
template <typename T, typename Op> __device__ __forceinline__ T reduce64(T v, Op op) {
  v = reduce16(v, op);
  T e, o;
  row_pair<16>(v, e, o);
  v = op(e, o);
  row_pair<32>(v, e, o);
  return op(e, o);
}
// lane and lane ^ 32 combined
template <typename T, typename Op> __device__ __forceinline__ T reduce_pair32(T v, Op op) {
  T e, o;
  row_pair<32>(v, e, o);
  return op(e, o);
}

struct OpMax {
  template <typename T> __device__ __forceinline__ T operator()(T a, T b) const {
    if constexpr (sizeof(T) == 8 && __is_same(T, double)) return fmax(a, b);
    else if constexpr (__is_same(T, float)) return fmaxf(a, b);
    else return a > b ? a : b;
  }
};
struct OpMin {
  template <typename T> __device__ __forceinline__ T operator()(T a, T b) const { return a < b ? a : b; }
};
struct OpSum {
  template <typename T> __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};

// 64-lane reductions (every lane receives the result).
template <typename T> __device__ __forceinline__ T wave_max(T v) { return reduce64(v, OpMax{}); }
template <typename T> __device__ __forceinline__ T wave_sum(T v) { return reduce64(v, OpSum{}); }
__device__ __forceinline__ int wave_min_int(int v) { return reduce64(v, OpMin{}); }
// 16-lane reductions (rows of 16 lanes)
template <typename T> __device__ __forceinline__ T group16_max(T v) { return reduce16(v, OpMax{}); }
template <typename T> __device__ __forceinline__ T group16_sum(T v) { return reduce16(v, OpSum{}); }

// Largest value; among equal values the lowest index.  Value and index travel
// together, so the pair reduction is the same total order in every lane.
struct ArgMax {
  double v;
  int i;
};
__device__ __forceinline__ ArgMax argmax_op(ArgMax a, ArgMax b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}
template <int CTRL> __device__ __forceinline__ ArgMax dpp_argmax(ArgMax a) {
  return ArgMax{dpp<CTRL>(a.v), dpp<CTRL>(a.i)};
}
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  ArgMax a{v, i};
  a = argmax_op(a, dpp_argmax<kDppXor1>(a));
  a = argmax_op(a, dpp_argmax<kDppXor2>(a));
  a = argmax_op(a, dpp_argmax<kDppHalfMirror>(a));
  a = argmax_op(a, dpp_argmax<kDppMirror>(a));
  ArgMax e, o;
  row_pair<16>(a.v, e.v, o.v), row_pair<16>(a.i, e.i, o.i);
  a = argmax_op(e, o);
  row_pair<32>(a.v, e.v, o.v), row_pair<32>(a.i, e.i, o.i);
  a = argmax_op(e, o);
  v = a.v, i = a.i;
}

__device__ __forceinline__ void flag_status(uint32_t* status, uint32_t bit) {
  atomicOr(status, bit);
}

// Token id checked against [0, V): out-of-range ids are reported and clamped.
__device__ __forceinline__ int checked_token(int x, int V, uint32_t* status, uint32_t bit) {
  if (x < 0 || x >= V) {
    flag_status(status, bit);
    return x < 0 ? 0 : V - 1;
  }
  return x;
}

// Temperatures below 2^-64 count as 0 (greedy), and so do NaN and negative
// values, which checked_temp() also reports.
__device__ __forceinline__ float effective_temp(float T) { return T >= 0x1p-64f ? T : 0.0f; }

__device__ __forceinline__ float checked_temp(float T, uint32_t* status) {
  if (!(T >= 0.0f)) flag_status(status, kBadTemp);
  return effective_temp(T);
}

// An index produced by a reduction that found no candidate (only possible with
// non-finite inputs) is replaced by `fallback` so that no access leaves its buffer.
__device__ __forceinline__ int index_or(int i, int limit, int fallback) {
  return (i >= 0 && i < limit) ? i : fallback;
}

// The chosen tile's 64 dot products U[prev] . W[v] (bf16 factors, r = 64 nj
// with nj = 2 or 4) in fp64 from exact bf16 x bf16 products, by a workgroup of
// 8 / NH wavefronts.  Lane l of wavefront w takes the rows v0 + 8 NH w +
// (l >> 3) + 8 h (h < NH) of W and the 16-byte chunks (l & 7) + 8 j of each, so
// that every load instruction reads eight whole 128-byte lines; load_h()
// fetches the matching U[prev] chunks.  Eight lanes then sum a row's partials,
// and every lane of the eight returns row h in out[h].
struct TileDot {
  static constexpr int kMaxJ = 4;
  uint4 hq[kMaxJ];
  int nj;
  __device__ __forceinline__ void load_h(const uint16_t* h, int lane) {
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j)
      if (j < nj) hq[j] = reinterpret_cast<const uint4*>(h)[(lane & 7) + 8 * j];
  }
  template <int NH = 2>
  __device__ __forceinline__ void dot(const uint16_t* W, int v0, int V, int wave, int lane, double (&out)[2]) const {
    uint4 wv[NH][kMaxJ];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int v = min(v0 + 8 * NH * wave + (lane >> 3) + 8 * hh, V - 1);
      const uint4* row = reinterpret_cast<const uint4*>(W + (size_t)v * (64 * nj));
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j)
        if (j < nj) wv[hh][j] = row[(lane & 7) + 8 * j];
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      // a product of two bf16 values is exact in fp32; the sum runs in fp64
      double c[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) {
        if (j >= nj) break;
        const uint32_t hv[4] = {hq[j].x, hq[j].y, hq[j].z, hq[j].w};
        const uint32_t ww[4] = {wv[hh][j].x, wv[hh][j].y, wv[hh][j].z, wv[hh][j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] += (double)(__uint_as_float(hv[q] << 16) * __uint_as_float(ww[q] << 16));
          c[q] += (double)(__uint_as_float(hv[q] & 0xffff0000u) * __uint_as_float(ww[q] & 0xffff0000u));
        }
      }
      double t = (c[0] + c[1]) + (c[2] + c[3]);
      t += __shfl_xor(t, 1);
      t += __shfl_xor(t, 2);
      t += __shfl_xor(t, 4);
      out[hh] = t;
    }
  }
};

}  // namespace dspark

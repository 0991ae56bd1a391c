// Packing of the Markov head's second factor W2 ("DSpark, la bozza che sa
// quando fermarsi", section "Un po' di autoregressione basta": B = W1 W2, W2 of
// r rows by V columns) into the vocabulary-major layout the round reads: row v
// of the packed matrix is column v of W2, so the r values that one vocabulary
// column contracts over are contiguous.  A static weight is packed once.
//
// One workgroup of 256 threads moves a 64 x 64 tile through LDS: reads along V
// (a row segment of W2 per wavefront pass), writes along r.
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kPT = 64;

template <typename T>
__global__ __launch_bounds__(256) void pack_w2_kernel(const T* __restrict__ w, T* __restrict__ out, int V, int r) {
  __shared__ T tile[kPT][kPT + 1];
  const int v0 = blockIdx.x * kPT, k0 = blockIdx.y * kPT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kPT; i += 4) {
    const int k = k0 + i, v = v0 + tx;
    if (k < r && v < V) tile[i][tx] = w[(size_t)k * V + v];
  }
  __syncthreads();
  for (int i = ty; i < kPT; i += 4) {
    const int v = v0 + i, k = k0 + tx;
    if (v < V && k < r) out[(size_t)v * r + k] = tile[tx][i];
  }
}

}  // namespace

hipError_t launch_pack_w2(const void* w, void* out, int elem_bytes, int V, int r, hipStream_t s) {
  const dim3 grid((V + kPT - 1) / kPT, (r + kPT - 1) / kPT);
  if (elem_bytes == 2)
    pack_w2_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out), V, r);
  else
    pack_w2_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(w), static_cast<float*>(out), V, r);
  return hipGetLastError();
}

}  // namespace dspark

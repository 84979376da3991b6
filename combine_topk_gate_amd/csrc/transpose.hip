// Batched transpose for weight preparation: src [batch, rows, cols] ->
// dst [batch, cols, rows], bf16 or f32.
//
// The layer stores every weight matrix with its reduction index contiguous
// (W_gate, W_up as [EL, F, H]; W_down as [EL, H, F]), the operand layout the
// matrix cores read on both sides of each product.  A caller holding the
// matrices as the math writes them (x W_gate with W_gate of H x F) converts
// them once with this, before the first layer call.  Not on the hot path.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kTrTile = 64;

// Each workgroup walks 64 x 64 tiles: 256 threads load a tile row by row in
// 16-byte vectors (coalesced), stage it in LDS with rows padded by one
// vector, and store it column by column in 16-byte vectors along the
// destination rows.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t batch,
                                                        int rows, int cols) {
  constexpr int V = 16 / sizeof(T);    // elements per vector: 8 (bf16) or 4 (f32)
  constexpr int VPR = kTrTile / V;     // vectors per tile row
  constexpr int RPP = 256 / VPR;       // tile rows per pass
  constexpr int P = kTrTile + V;       // LDS pitch in elements
  typedef T vec_t __attribute__((ext_vector_type(V)));
  __shared__ __attribute__((aligned(16))) T tile[kTrTile * P];
  const int tr = rows / kTrTile, tc = cols / kTrTile;
  const int64_t tiles = batch * tr * tc;
  const int q = threadIdx.x % VPR, r = threadIdx.x / VPR;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t b = t / ((int64_t)tr * tc);
    const int rem = (int)(t - b * tr * tc);
    const int r0 = (rem / tc) * kTrTile, c0 = (rem % tc) * kTrTile;
    const T* s = src + (b * rows + r0) * (int64_t)cols + c0;
    for (int i = r; i < kTrTile; i += RPP)
      *reinterpret_cast<vec_t*>(&tile[i * P + q * V]) = *reinterpret_cast<const vec_t*>(s + (int64_t)i * cols + q * V);
    __syncthreads();
    T* d = dst + (b * cols + c0) * (int64_t)rows + r0;
    for (int o = r; o < kTrTile; o += RPP) {
      vec_t v;
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = tile[(q * V + e) * P + o];
      *reinterpret_cast<vec_t*>(d + (int64_t)o * rows + q * V) = v;
    }
    __syncthreads();
  }
}

hipError_t launch_transpose(const void* src, void* dst, int64_t batch, int rows, int cols, bool bf16, hipStream_t s) {
  const int64_t tiles = batch * (rows / kTrTile) * (int64_t)(cols / kTrTile);
  if (tiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)(tiles < 4096 ? tiles : 4096);
  if (bf16)
    transpose_kernel<__bf16><<<grid, 256, 0, s>>>(reinterpret_cast<const __bf16*>(src), reinterpret_cast<__bf16*>(dst),
                                                  batch, rows, cols);
  else
    transpose_kernel<float><<<grid, 256, 0, s>>>(reinterpret_cast<const float*>(src), reinterpret_cast<float*>(dst),
                                                 batch, rows, cols);
  return hipGetLastError();
}

}  // namespace moe

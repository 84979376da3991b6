// Top-k weighted combine.
//
// COMET paper review §4.1.1 (the Layer1 consumer is the Top-K reduction,
// which couples the k rows of a token, so Layer1's shared tensor splits
// along N) and the PTO MoE article (Combine + Unpermute: top-K weighted
// accumulation back into token order).
//   out[t, n] = sum_{j<k} w[t,j] * Y[flat_to_sorted[t*k+j], n]
// in f32, from zero, j increasing, one fused multiply-add per term, over
// the slots whose pair is held here; then the epilogue (optional residual
// add, f32 or bf16 output).
// A block walks whole token rows, 4 columns per lane per step, so every
// Y row read and every out row write is contiguous.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ y,
                                                                  const float* __restrict__ topk_w,
                                                                  const int32_t* __restrict__ f2s, int64_t M, int H,
                                                                  int k, OutEpilogue ep) {
  __shared__ int rows[16];
  __shared__ float w[16];
  const int groups = H / 4;
  for (int64_t t = blockIdx.x; t < M; t += gridDim.x) {
    if (threadIdx.x < k) {
      rows[threadIdx.x] = f2s[t * k + threadIdx.x];
      w[threadIdx.x] = topk_w[t * k + threadIdx.x];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < groups; q += kCombineThreads) {
      const float4 o = combine_group(y, w, rows, k, H, (int64_t)q * 4);
      store_out(ep, t * H + (int64_t)q * 4, o);
    }
    __syncthreads();
  }
}

hipError_t launch_combine(const float* y, const float* topk_w, const int32_t* flat_to_sorted, int64_t M, int H,
                          int k, const OutEpilogue& ep, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t grid = M < 16384 ? M : 16384;
  combine_kernel<<<(unsigned)grid, kCombineThreads, 0, s>>>(y, topk_w, flat_to_sorted, M, H, k, ep);
  return hipGetLastError();
}

}  // namespace moe

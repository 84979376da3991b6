// Top-k weighted combine.
//
// COMET paper review §4.1.1 (the Layer1 consumer is the Top-K reduction,
// which couples the k rows of a token, so Layer1's shared tensor splits
// along N) and the PTO MoE article (Combine + Unpermute: top-K weighted
// accumulation back into token order).
//   out[t, n] = sum_{j<k} w[t,j] * Y[flat_to_sorted[t*k+j], n]
// in f32, from zero, j increasing, one fused multiply-add per term, over
// the slots whose pair is held here (a row index outside [0, M k) counts as
// not held); then the epilogue (optional residual add, f32 or bf16 output).
// A block walks whole token rows, 4 columns per lane per step, so every
// Y row read and every out row write is contiguous.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kCombineUnroll = 4;

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
    // kCombineUnroll column groups per thread at a time, two slots per
    // step: both slots' loads for all of them are issued before any is used
    // (the per-element arithmetic is combine_group's: from zero, slots in
    // order, fmaf)
    for (int q0 = threadIdx.x; q0 < groups; q0 += kCombineThreads * kCombineUnroll) {
      float4 acc[kCombineUnroll];
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j0 = 0; j0 < k; j0 += 2) {
        float4 v[2][kCombineUnroll];
        bool held[2];
        float wj[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = j0 + h;
          const int32_t row = j < k ? rows[j] : -1;
          held[h] = (uint64_t)(int64_t)row < (uint64_t)(M * k);  // -1: a pair of an expert not held here
          wj[h] = held[h] ? w[j] : 0.f;
          const float* yr = y + (int64_t)(held[h] ? row : 0) * H;
#pragma unroll
          for (int u = 0; u < kCombineUnroll; ++u) {
            const int q = q0 + u * kCombineThreads;
            v[h][u] = held[h] && q < groups ? *reinterpret_cast<const float4*>(yr + (int64_t)q * 4)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (!held[h]) continue;
#pragma unroll
          for (int u = 0; u < kCombineUnroll; ++u) {
            acc[u].x = fmaf(wj[h], v[h][u].x, acc[u].x);
            acc[u].y = fmaf(wj[h], v[h][u].y, acc[u].y);
            acc[u].z = fmaf(wj[h], v[h][u].z, acc[u].z);
            acc[u].w = fmaf(wj[h], v[h][u].w, acc[u].w);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const int q = q0 + u * kCombineThreads;
        if (q < groups) store_out(ep, t * H + (int64_t)q * 4, acc[u]);
      }
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

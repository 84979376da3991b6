// Top-k routing with renormalised softmax weights.
//
// COMET paper review §4.1.1 (Top-K reduction couples a token's expert
// outputs) and the PTO MoE article's seven serial stages (top-K weighted
// accumulation): each token keeps its k largest gate logits, and the
// weights are the softmax over the k chosen logits.
//
// One wave handles 64 tokens, one token per lane.  The wave stages its
// 64 x E logits through LDS in chunks of 64 experts so the HBM reads are
// coalesced, then every lane walks its row in increasing expert order and
// keeps the KMAX best (value, index) pairs sorted in registers.  A new value
// enters only if it is strictly greater than the current KMAX-th value and
// goes behind every kept value it does not exceed, so equal logits keep the
// lower index first.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRouteTokens = 64;
constexpr int kRouteChunk = 64;

template <int KMAX>
__device__ __forceinline__ void topk_insert(float (&vals)[KMAX], int (&ids)[KMAX], float v, int e) {
  if (!(v > vals[KMAX - 1])) return;
#pragma unroll
  for (int i = KMAX - 1; i >= 0; --i) {
    // position i keeps its value if that value is >= v; otherwise it takes
    // v (if the slot above it is >= v, or i == 0) or the value from above.
    if (vals[i] >= v) continue;
    const bool above_ge = (i == 0) ? true : (vals[i - 1] >= v);
    if (above_ge) {
      vals[i] = v;
      ids[i] = e;
    } else {
      vals[i] = vals[i - 1];
      ids[i] = ids[i - 1];
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(kRouteTokens) void route_topk_kernel(const float* __restrict__ logits, int64_t M, int E,
                                                                   int k, int32_t* __restrict__ topk_idx,
                                                                   float* __restrict__ topk_w) {
  __shared__ float tile[kRouteTokens][kRouteChunk + 1];
  const int lane = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTokens;
  const int ntok = (int)((M - t0) < kRouteTokens ? (M - t0) : kRouteTokens);

  float vals[KMAX];
  int ids[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    vals[i] = -__builtin_inff();
    ids[i] = 0;
  }

  for (int c0 = 0; c0 < E; c0 += kRouteChunk) {
    const int ce = (E - c0) < kRouteChunk ? (E - c0) : kRouteChunk;
    const int n = ntok * ce;
    for (int i = lane; i < n; i += kRouteTokens) {
      const int tt = i / ce, ee = i - tt * ce;
      tile[tt][ee] = logits[(t0 + tt) * (int64_t)E + c0 + ee];
    }
    __syncthreads();
    if (lane < ntok) {
      for (int ee = 0; ee < ce; ++ee) topk_insert<KMAX>(vals, ids, tile[lane][ee], c0 + ee);
    }
    __syncthreads();
  }
  if (lane >= ntok) return;

  const int64_t t = t0 + lane;
  const float l0 = vals[0];
  float denom = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) denom += expf(vals[j] - l0);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      topk_idx[t * k + j] = ids[j];
      topk_w[t * k + j] = expf(vals[j] - l0) / denom;
    }
  }
}

hipError_t launch_route(const float* logits, int64_t M, int E, int k, int32_t* topk_idx, float* topk_w,
                        hipStream_t s) {
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)((M + kRouteTokens - 1) / kRouteTokens)), block(kRouteTokens);
  if (k <= 1)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w);
  else if (k <= 2)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w);
  else if (k <= 4)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w);
  else if (k <= 8)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w);
  else
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe

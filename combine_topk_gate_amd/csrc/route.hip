// Top-k routing with renormalised softmax weights.
//
// COMET paper review §4.1.1 (Top-K reduction couples a token's expert
// outputs) and the PTO MoE article's seven serial stages (top-K weighted
// accumulation): each token keeps its k largest gate logits, and the
// weights are the softmax over the k chosen logits.
//
// Sixteen lanes handle one token (a 256-thread block: 16 tokens).  Lane q
// reads experts q, q + 16, q + 32, ... (the 16 lanes of a token read 64
// consecutive bytes at a time) and keeps its KMAX best (value, index) pairs
// sorted in registers.  The lanes' lists are then merged in four butterfly
// steps: partners exchange their lists and both keep the KMAX best of the
// union.  "Best" is the total order value descending, then index ascending,
// which is the order the selection defines (equal logits keep the lower
// expert index first), so the merged list is unique and every lane of the
// token ends with the same one.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kLanesPerToken = 16;

// a ahead of b: larger value, or equal value and lower index
__device__ __forceinline__ bool route_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int KMAX>
__device__ __forceinline__ void topk_insert(float (&vals)[KMAX], int (&ids)[KMAX], float v, int e) {
  // e exceeds every index kept so far, so v enters only if strictly larger
  // than the last kept value, behind every kept value it does not exceed
  if (!(v > vals[KMAX - 1])) return;
#pragma unroll
  for (int i = KMAX - 1; i >= 0; --i) {
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

// Keep the KMAX best of two sorted lists (own and the partner lane's):
// pairing own[i] with partner[KMAX-1-i] and keeping the better of each pair
// leaves the KMAX best as a bitonic sequence, which a bitonic merger sorts.
template <int KMAX>
__device__ __forceinline__ void topk_merge_partner(float (&vals)[KMAX], int (&ids)[KMAX], int off) {
  float pv[KMAX];
  int pi[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    pv[i] = __shfl_xor(vals[i], off);
    pi[i] = __shfl_xor(ids[i], off);
  }
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const float bv = pv[KMAX - 1 - i];
    const int bi = pi[KMAX - 1 - i];
    if (!route_before(vals[i], ids[i], bv, bi)) {
      vals[i] = bv;
      ids[i] = bi;
    }
  }
#pragma unroll
  for (int half = KMAX / 2; half >= 1; half >>= 1) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i & half) continue;
      const int j = i + half;
      if (!route_before(vals[i], ids[i], vals[j], ids[j])) {
        const float tv = vals[i];
        const int ti = ids[i];
        vals[i] = vals[j];
        ids[i] = ids[j];
        vals[j] = tv;
        ids[j] = ti;
      }
    }
  }
}

// Words the caller needs zero before the kernels that follow (the layer
// call's status word and the fused kernel's ready counters): block 0 clears
// them, which saves a launch per range.
struct ClearRanges {
  int32_t* p0 = nullptr;
  int n0 = 0;
  int32_t* p1 = nullptr;
  int n1 = 0;
};

template <int KMAX>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float* __restrict__ logits, int64_t M, int E,
                                                                   int k, int32_t* __restrict__ topk_idx,
                                                                   float* __restrict__ topk_w, ClearRanges clr) {
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < clr.n0; i += kRouteThreads) clr.p0[i] = 0;
    for (int i = threadIdx.x; i < clr.n1; i += kRouteThreads) clr.p1[i] = 0;
  }
  const int q = threadIdx.x % kLanesPerToken;
  const int64_t t = (int64_t)blockIdx.x * (kRouteThreads / kLanesPerToken) + threadIdx.x / kLanesPerToken;
  const bool valid = t < M;  // whole 16-lane groups share `valid`
  float vals[KMAX];
  int ids[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    vals[i] = -__builtin_inff();
    ids[i] = 0x7fffffff;  // behind every real expert (logits are finite)
  }
  if (valid) {
    const float* row = logits + t * (int64_t)E;
    // 4 loads in flight per lane, then insertion in increasing expert order
    int e = q;
    for (; e + 3 * kLanesPerToken < E; e += 4 * kLanesPerToken) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = row[e + u * kLanesPerToken];
#pragma unroll
      for (int u = 0; u < 4; ++u) topk_insert<KMAX>(vals, ids, v[u], e + u * kLanesPerToken);
    }
    for (; e < E; e += kLanesPerToken) topk_insert<KMAX>(vals, ids, row[e], e);
  }
#pragma unroll
  for (int off = 1; off < kLanesPerToken; off <<= 1) topk_merge_partner<KMAX>(vals, ids, off);
  if (!valid) return;

  // weights: softmax over the k chosen logits, shifted by the largest,
  // summed in slot order; lane j < k writes slot j
  const float l0 = vals[0];
  float denom = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) denom += expf(vals[j] - l0);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && j == q) {
      topk_idx[t * k + j] = ids[j];
      topk_w[t * k + j] = expf(vals[j] - l0) / denom;
    }
  }
}

hipError_t launch_route(const float* logits, int64_t M, int E, int k, int32_t* topk_idx, float* topk_w,
                        hipStream_t s, int32_t* clear0, int n0, int32_t* clear1, int n1) {
  if (M == 0) return hipSuccess;
  ClearRanges clr;
  clr.p0 = clear0;
  clr.n0 = clear0 ? n0 : 0;
  clr.p1 = clear1;
  clr.n1 = clear1 ? n1 : 0;
  const int64_t per_block = kRouteThreads / kLanesPerToken;
  const dim3 grid((unsigned)((M + per_block - 1) / per_block)), block(kRouteThreads);
  if (k <= 1)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w, clr);
  else if (k <= 2)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w, clr);
  else if (k <= 4)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w, clr);
  else if (k <= 8)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w, clr);
  else
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, M, E, k, topk_idx, topk_w, clr);
  return hipGetLastError();
}

}  // namespace moe

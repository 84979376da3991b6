// Host-side launchers of the library's kernels (internal; the public entry
// points in api.hip validate arguments and call these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

hipError_t launch_route(const float* logits, int64_t M, int E, int k, int32_t* topk_idx, float* topk_w,
                        hipStream_t s);

// Segment bookkeeping: per-chunk histograms, scan, stable ranks.  Pairs of
// experts outside [base, base + EL) are dropped: they form an extra last
// segment (index G) inside the bookkeeping, which is not reported.
struct PermutePlan {
  int64_t R;
  int G;       // segments reported: S * EL
  int Gi;      // segments ranked: G, or G + 1 when some experts are not held
  int EL;      // experts held
  int base;    // first expert held
  int chunk;   // pairs per block
  int blocks;  // ceil(R / chunk)
};
PermutePlan permute_plan(int64_t M, int k, int S, int E, int base, int EL);
size_t permute_ws_bytes(const PermutePlan& pl);
hipError_t launch_permute(const PermutePlan& pl, const int32_t* topk_idx, const int32_t* src_block, int k,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                          int32_t* ws, hipStream_t s);
// Rows of dropped pairs (flat_to_sorted -1) are not written.
hipError_t launch_dispatch_copy(const void* x, int64_t M, int64_t row_bytes, int k, const int32_t* flat_to_sorted,
                                void* x_perm, hipStream_t s);

// Grouped GEMM (layer 0: gate/up + SwiGLU; layer 1: down).
struct GemmProblem {
  int layer;
  const void* a;
  const void* w0;
  const void* w1;
  const int32_t* offsets;
  void* c;
  int64_t R;
  int K;  // reduction length: H (layer 0) or F (layer 1)
  int N;  // output columns: F (layer 0) or H (layer 1)
  int E;
  int G;
  void* ws = nullptr;       // bf16: split workspace of gemm_split_ws_bytes(), or null
  size_t ws_bytes = 0;
};
// Workspace that lets the bf16 grouped GEMM split its last round along K.
size_t gemm_split_ws_bytes();
hipError_t launch_grouped_gemm_bf16(const GemmProblem& gp, hipStream_t s);
hipError_t launch_grouped_gemm_f32(const GemmProblem& gp, hipStream_t s);
// MXFP8 activation path: layer 0 bf16 -> Hact MXFP8; layer 1 MXFP8 x MXFP8 -> Y.
// An MXFP8 tensor of rows x cols is one buffer: codes, then cols/32 scale
// bytes per row.
hipError_t launch_grouped_gemm_mx(const GemmProblem& gp, hipStream_t s);
hipError_t launch_mx_quantize(const void* src, int src_bf16, int64_t rows, int cols, void* dst, hipStream_t s);

hipError_t launch_combine(const float* y, const float* topk_w, const int32_t* flat_to_sorted, int64_t M, int H,
                          int k, const OutEpilogue& ep, hipStream_t s);

int device_cu_count();

}  // namespace moe

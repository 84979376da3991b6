// Host-side launchers of the library's kernels (internal; the public entry
// points in api.hip validate arguments and call these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

// clear0 / clear1 (n0 / n1 words, null for none): words the kernel's first
// block sets to zero, for kernels launched after it (the layer call's status
// word and the fused kernel's ready counters), instead of a fill launch each.
hipError_t launch_route(const float* logits, int64_t M, int E, int k, int32_t* topk_idx, float* topk_w,
                        hipStream_t s, int32_t* clear0 = nullptr, int n0 = 0, int32_t* clear1 = nullptr,
                        int n1 = 0);

// Dispatch: segment bookkeeping (per-chunk histograms, bases, stable ranks)
// and the copy of token rows to their sorted positions.  Pairs of experts
// outside [base, base + EL) are dropped: they form an extra last segment
// (index G) inside the bookkeeping, which is not reported.
struct PermutePlan {
  int64_t M;
  int k;
  int64_t R;
  int G;        // segments reported: S * EL
  int Gi;       // segments ranked: G, or G + 1 when some experts are not held
  int EL;       // experts held
  int base;     // first expert held
  int Tc;       // tokens per chunk (a histogram each)
  int Ts;       // tokens per dispatch workgroup
  int blocks;   // chunks: ceil(M / Tc)
  int64_t wgs;  // dispatch workgroups: ceil(M / Ts)
  int scanned;  // a scan kernel turns the histograms into bases first
};
PermutePlan permute_plan(int64_t M, int k, int S, int E, int base, int EL);
size_t permute_ws_bytes(const PermutePlan& pl);
// Device address of this GPU's static scratch (MOE_NOALLOC_SCRATCH_BYTES),
// looked up on the first call on each device.
hipError_t static_scratch(void** addr);
// x_perm null: the bookkeeping only (x is not read).  Rows of dropped pairs
// (flat_to_sorted -1) are not written.
hipError_t launch_dispatch(const PermutePlan& pl, const int32_t* topk_idx, const int32_t* src_block,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                           const void* x, int64_t row_bytes, void* x_perm, int32_t* ws, hipStream_t s);

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
  int rowmap = 0;           // bf16: each expert's segments of all source blocks as one (G / E of them)
  uint32_t shuffle = 0;     // nonzero: tiles in a seeded permutation of their order (debug check)
};
// Workspace that lets the bf16 grouped GEMM split its last round along K.
size_t gemm_split_ws_bytes();
hipError_t launch_grouped_gemm_bf16(const GemmProblem& gp, hipStream_t s);
hipError_t launch_grouped_gemm_f32(const GemmProblem& gp, hipStream_t s);
// MXFP8 activation path: layer 0 bf16 -> Hact MXFP8; layer 1 MXFP8 x MXFP8 -> Y.
// An MXFP8 tensor of rows x cols (cols a multiple of 128) is one buffer: the
// rows*cols codes, then the scale bytes in groups of 32 rows (rows padded to
// a multiple of 32): the byte of row r, block b sits at
// (r / 32) * cols + (b / 4) * 128 + (r % 32) * 4 + b % 4.
hipError_t launch_grouped_gemm_mx(const GemmProblem& gp, hipStream_t s);
hipError_t launch_mx_quantize(const void* src, int src_bf16, int64_t rows, int cols, void* dst, hipStream_t s);
// Batched transpose src [batch, rows, cols] -> dst [batch, cols, rows]; rows
// and cols multiples of 64; bf16 (else f32) elements.
hipError_t launch_transpose(const void* src, void* dst, int64_t batch, int rows, int cols, bool bf16, hipStream_t s);

hipError_t launch_combine(const float* y, const float* topk_w, const int32_t* flat_to_sorted, int64_t M, int H,
                          int k, const OutEpilogue& ep, hipStream_t s);

int device_cu_count();

}  // namespace moe

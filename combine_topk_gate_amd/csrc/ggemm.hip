// Persistent grouped-GEMM kernels: bf16 (matrix cores) and f32 (vector FMA).
//
// "Grouped GEMM 为什么适合 MoE": a fixed number of workgroups walks one
// tile queue spanning every expert problem, instead of one launch per
// expert.  Here the queue is static: workgroup slot v takes tiles v,
// v + grid, v + 2 grid, ... of the order tiles.hpp defines, so the
// schedule needs no counter in memory and the tile-to-workgroup map is a
// pure function of the offsets.
#include "common.hpp"
#include "gemm_bf16.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

// The grid's last round is re-cut: when its r tiles would fill at most half
// the workgroups, they become 2 r half tiles (128 token rows each), so the
// round takes about half a tile's time instead of a whole one.  A half tile
// computes each element exactly as a full tile does (same k order), so the
// split never changes the result.  (Measured on MI355X: halving the tail
// tile of every segment instead costs more than the padding it saves.)
template <int LAYER>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(Bf16GemmArgs args,
                                                                         const int32_t* __restrict__ offsets, int G,
                                                                         int group_cols) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLdsBytes];
  __shared__ TileLds tl;
  const int NT = (args.N + (LAYER == 0 ? kL0Cols : kL1Cols) - 1) / (LAYER == 0 ? kL0Cols : kL1Cols);
  const int T = build_tile_table(offsets, G, kTileRows, tl) * NT;
  const int grid = gridDim.x;
  const int r = T % grid;
  const int split = (r > 0 && 2 * r <= grid && T > grid) ? r : 0;  // tiles of the last round to halve
  const int entries = T + split;
  for (int v = xcd_slot(blockIdx.x, grid); v < entries; v += grid) {
    if (v < T - split) {
      const TileCoord c = tile_coord(v, G, NT, kTileRows, group_cols, tl);
      bf16_gemm_tile<LAYER>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
    } else {
      const int j = v - (T - split);
      const TileCoord c = tile_coord(T - split + j / 2, G, NT, kTileRows, group_cols, tl);
      const int m0 = c.m0 + (j & 1) * (kTileRows / 2);
      if (m0 < tl.seg_rows[c.g]) bf16_gemm_tile<LAYER, false, kTileRows / 2>(args, c.g, tl.seg_start[c.g],
                                                                              tl.seg_rows[c.g], m0, c.nt, lds);
    }
  }
}

// ------------------------------------------------------------------ f32 ---
// Small-layer path in f32 (no reduced-precision matrix mode): 64 token rows
// x 64 weight rows per tile, K stepped by 32 through LDS, each thread a 4 x 4
// block accumulated with fmaf in increasing k.  Layer0's 64 weight rows are
// 32 gate and the matching 32 up rows.
constexpr int kF32Rows = 64;
constexpr int kF32BK = 32;

template <int LAYER>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                               const float* __restrict__ W0,
                                                               const float* __restrict__ W1, float* __restrict__ C,
                                                               int K, int N, int E, const int32_t* __restrict__ offsets,
                                                               int G) {
  __shared__ float xs[kF32Rows][kF32BK + 1];
  __shared__ float ws[kF32Rows][kF32BK + 1];
  __shared__ TileLds tl;
  constexpr int cols = (LAYER == 0) ? kF32Rows / 2 : kF32Rows;
  const int NT = (N + cols - 1) / cols;
  const int total = build_tile_table(offsets, G, kF32Rows, tl) * NT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int v = blockIdx.x; v < total; v += gridDim.x) {
    const TileCoord c = tile_coord(v, G, NT, kF32Rows, 1, tl);
    const int e = c.g % E, s0 = tl.seg_start[c.g], nrows = tl.seg_rows[c.g];
    const int col0 = c.nt * cols;
    const int64_t ebase = (int64_t)e * N * K;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kF32BK) {
      for (int i = tid; i < kF32Rows * kF32BK; i += 256) {
        const int r = i / kF32BK, kk = i % kF32BK;
        const int tr = c.m0 + r;
        xs[r][kk] = (tr < nrows) ? A[(int64_t)(s0 + tr) * K + k0 + kk] : 0.0f;
        int wr, wcol;
        const float* W;
        if (LAYER == 0) {
          W = (r < 32) ? W0 : W1;
          wcol = col0 + (r & 31);
        } else {
          W = W0;
          wcol = col0 + r;
        }
        wr = wcol;
        ws[r][kk] = (wr < N) ? W[ebase + (int64_t)wr * K + k0 + kk] : 0.0f;
      }
      __syncthreads();
      for (int kk = 0; kk < kF32BK; ++kk) {
        float wv[4], xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[i] = ws[tx + 16 * i][kk];
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = xs[ty + 16 * j][kk];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(wv[i], xv[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tr = c.m0 + ty + 16 * j;
      if (tr >= nrows) continue;
      float* dst = C + (int64_t)(s0 + tr) * N;
      if (LAYER == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int f = col0 + tx + 16 * i;
          if (f < N) dst[f] = silu_f32(acc[i][j]) * acc[i + 2][j];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = col0 + tx + 16 * i;
          if (n < N) dst[n] = acc[i][j];
        }
      }
    }
  }
}

static int g_cu_count = 0;

int device_cu_count() {
  if (g_cu_count == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && n > 0)
      g_cu_count = n;
    else
      g_cu_count = 256;
  }
  return g_cu_count;
}

hipError_t launch_grouped_gemm_bf16(const GemmProblem& gp, hipStream_t s) {
  if (gp.R == 0) return hipSuccess;
  Bf16GemmArgs a;
  a.a = (const __bf16*)gp.a;
  a.w0 = (const __bf16*)gp.w0;
  a.w1 = (const __bf16*)gp.w1;
  a.c = gp.c;
  a.K = gp.K;
  a.N = gp.N;
  a.E = gp.E;
  a.s2f = nullptr;
  a.topk = 1;
  a.M = 0;
  const int grid = device_cu_count();
  const int group_cols = grid / kXcds > 0 ? grid / kXcds : 1;
  if (gp.layer == 0)
    grouped_gemm_bf16_kernel<0><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, group_cols);
  else
    grouped_gemm_bf16_kernel<1><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, group_cols);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_f32(const GemmProblem& gp, hipStream_t s) {
  if (gp.R == 0) return hipSuccess;
  const int grid = device_cu_count() * 2;
  if (gp.layer == 0)
    grouped_gemm_f32_kernel<0><<<grid, 256, 0, s>>>((const float*)gp.a, (const float*)gp.w0, (const float*)gp.w1,
                                                     (float*)gp.c, gp.K, gp.N, gp.E, gp.offsets, gp.G);
  else
    grouped_gemm_f32_kernel<1><<<grid, 256, 0, s>>>((const float*)gp.a, (const float*)gp.w0, nullptr,
                                                    (float*)gp.c, gp.K, gp.N, gp.E, gp.offsets, gp.G);
  return hipGetLastError();
}

}  // namespace moe

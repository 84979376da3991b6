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
#include "gemm_mx.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

// Workspace of a split last round: header {r, s} and one descriptor
// {seg_start, seg_rows, m0, nt} per split tile, then the partial
// accumulators, one 256 x 256 f32 block per unit (at most one unit per CU).
struct SplitWs {
  int32_t* hdr;
  int32_t* desc;
  float* part;
};
constexpr int kMaxSplit = 8;
constexpr int kMinSplitSteps = 4;  // K steps per range, at least
constexpr size_t kSplitPartFloats = (size_t)kTileRows * 256;
constexpr size_t kSplitHdrBytes = 16 + 16 * 4096;  // descriptors of up to 4096 split tiles

// Whether splitting a last-round tile of nk K steps into s ranges shortens
// the round, in units of one K step of a full tile: the half-tile tail
// (halfable) takes about 0.55 nk (half the MFMAs, the same operand loads
// per K step of the weights), an unsplit full tile nk, a split one nk / s
// plus the partial stores and the reduce pass, about 16 steps (measured on
// layer 1 with H = 4096: 256 KiB of f32 per unit written, read back once).
__device__ __forceinline__ bool split_pays(int nk, int s, bool halfable) {
  const int base = halfable ? 55 * nk : 100 * nk;
  return base - 100 * nk / s > 1600;
}

// The grid's last round is re-cut so that it ends sooner.
//  * Layer 1 with a split workspace (`split` non-null): its r tiles are cut
//    along K into s = min(grid / r, steps / kMinSplitSteps, kMaxSplit)
//    ranges each (when split_pays), r s <= grid units, every CU takes at
//    most one.  A unit stores its raw f32 accumulators (SplitWs::part) and
//    grouped_gemm_split_reduce adds the s ranges of each tile in increasing
//    order.  Layer 0 does not split: its tiles are 4 to 7 times shorter, so
//    the partials and the second pass cost about what the split saves, and
//    the split path's registers would raise the kernel's spills.
//  * Otherwise, when its r tiles would fill at most half the workgroups,
//    they become 2 r half tiles (128 token rows each), which compute each
//    element exactly as a full tile does.
// The split is a function of the tile count and the grid, so a given device
// always splits the same tiles the same way.
// OUT8 (layer 0): Hact is written in MXFP8 (codes to args.c, scales to
// args.c_scale) for the MXFP8 Layer1 below.
template <int LAYER, bool OUT8 = false>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(Bf16GemmArgs args,
                                                                         const int32_t* __restrict__ offsets, int G,
                                                                         int xcd_slots, SplitWs split,
                                                                         uint32_t shuffle) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLdsBytes];
  __shared__ TileLds tl;
  const int NT = (args.N + (LAYER == 0 ? kL0Cols : kL1Cols) - 1) / (LAYER == 0 ? kL0Cols : kL1Cols);
  const int T = build_tile_table(offsets, G, kTileRows, tl) * NT;
  const int64_t rtb = (int64_t)kTileRows * args.K * 2;  // bytes of a tile's operand panel (bf16)
  const int grid = gridDim.x;
  const int r = T % grid;
  if constexpr (LAYER == 1 && !OUT8) {
    const int nk = args.K / kBK;
    int s = 1;
    if (split.hdr && r > 0) s = min(min(grid / r, nk / kMinSplitSteps), kMaxSplit);
    if (s >= 2 && !split_pays(nk, s, 2 * r <= grid && T > grid)) s = 1;
    if (split.hdr && blockIdx.x == 0 && threadIdx.x == 0) {
      split.hdr[0] = s >= 2 ? r : 0;
      split.hdr[1] = s;
    }
    if (s >= 2) {
      const int tail0 = T - r;
      const int entries = tail0 + r * s;
      const Shuffle sm = make_shuffle(shuffle, tail0), st = make_shuffle(shuffle, r);
      for (int v = xcd_slot(blockIdx.x, grid); v < entries; v += grid) {
        if (v < tail0) {
          const TileCoord c = tile_coord(shuffled(sm, v), G, NT, kTileRows, xcd_slots, rtb, tl);
          bf16_gemm_row_tile<LAYER>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
        } else {
          const int u = v - tail0, jj = u / s, ck = u - jj * s;
          const TileCoord c = tile_coord(tail0 + shuffled(st, jj), G, NT, kTileRows, xcd_slots, rtb, tl);
          if (ck == 0 && threadIdx.x == 0) {
            int32_t* d = split.desc + 4 * jj;
            d[0] = tl.seg_start[c.g];
            d[1] = tl.seg_rows[c.g];
            d[2] = c.m0;
            d[3] = c.nt;
          }
          bf16_gemm_tile<LAYER, false, kTileRows, true>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt,
                                                        lds, (ck * nk) / s, ((ck + 1) * nk) / s,
                                                        split.part + (size_t)u * kSplitPartFloats);
        }
      }
      return;
    }
  }
  const int half = (r > 0 && 2 * r <= grid && T > grid) ? r : 0;  // tiles of the last round to halve
  const int entries = T + half;
  const Shuffle sm = make_shuffle(shuffle, T - half), sh = make_shuffle(shuffle, half);
  for (int v = xcd_slot(blockIdx.x, grid); v < entries; v += grid) {
    if (v < T - half) {
      const TileCoord c = tile_coord(shuffled(sm, v), G, NT, kTileRows, xcd_slots, rtb, tl);
      bf16_gemm_row_tile<LAYER, false, OUT8>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
    } else {
      const int j = v - (T - half);
      const TileCoord c = tile_coord(T - half + shuffled(sh, j / 2), G, NT, kTileRows, xcd_slots, rtb, tl);
      const int m0 = c.m0 + (j & 1) * (kTileRows / 2);
      if (m0 < tl.seg_rows[c.g])
        bf16_gemm_tile<LAYER, false, kTileRows / 2, false, OUT8>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], m0,
                                                                 c.nt, lds);
    }
  }
}

// The grouped GEMM over combined per-expert segments (GemmProblem::rowmap):
// when the rows arrive in many source blocks, the segment of one (source
// block, expert) pair can be far shorter than a tile (the expert-parallel
// share that holds 16 of 128 experts: about 128 rows each), so every
// weight panel would be streamed once per source block for half a tile of
// rows.  Here the S segments of expert e are one combined segment
// (build_expert_tile_table), and each tile looks up its rows' sorted
// positions once (expert_row, into LDS) for its loads and its stores.  The
// same static schedule and last-round halves as the kernel above; no split
// along k.  Every element is computed as in any other tile, so the bits do
// not change.
template <int LAYER>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_expert_kernel(Bf16GemmArgs args,
                                                                                const int32_t* __restrict__ offsets,
                                                                                int G, int xcd_slots,
                                                                                uint32_t shuffle) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLdsBytes];
  __shared__ TileLds tl;
  __shared__ int rowpos[kTileRows];
  const int EL = args.E, S = G / EL;
  const int NT = (args.N + (LAYER == 0 ? kL0Cols : kL1Cols) - 1) / (LAYER == 0 ? kL0Cols : kL1Cols);
  const int T = build_expert_tile_table(offsets, G, EL, kTileRows, tl) * NT;
  const int64_t rtb = (int64_t)kTileRows * args.K * 2;
  const int grid = gridDim.x;
  const int r = T % grid;
  const int half = (r > 0 && 2 * r <= grid && T > grid) ? r : 0;  // tiles of the last round to halve
  const int entries = T + half;
  const Shuffle sm = make_shuffle(shuffle, T - half), sh = make_shuffle(shuffle, half);
  for (int v = xcd_slot(blockIdx.x, grid); v < entries; v += grid) {
    const bool is_half = v >= T - half;
    const int j = v - (T - half);
    const TileCoord c = tile_coord(is_half ? T - half + shuffled(sh, j / 2) : shuffled(sm, v), EL, NT, kTileRows,
                                   xcd_slots, rtb, tl);
    const int m0 = is_half ? c.m0 + (j & 1) * (kTileRows / 2) : c.m0;
    const int n = tl.expert_rows[c.g];
    if (m0 >= n) continue;
    rowpos[threadIdx.x] = expert_row(tl, c.g, EL, S, m0, threadIdx.x);
    __syncthreads();
    if (is_half)
      bf16_gemm_tile<LAYER, false, kTileRows / 2, false, false, true>(args, c.g, 0, n, m0, c.nt, lds, 0, -1, nullptr,
                                                                      rowpos);
    else
      bf16_gemm_row_tile<LAYER, false, false, true>(args, c.g, 0, n, m0, c.nt, lds, rowpos);
  }
}

// Layer1 on MXFP8 operands: the same persistent schedule (tile order,
// half-height tiles for single-tile segments of at most 128 rows and for a
// last round that would leave more than half the CUs idle) with the MXFP8
// tile; no split of the last round.
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_mx_kernel(Bf16GemmArgs args,
                                                                       const int32_t* __restrict__ offsets, int G,
                                                                       int xcd_slots, uint32_t shuffle) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLdsBytes];
  __shared__ TileLds tl;
  const int NT = (args.N + kL1Cols - 1) / kL1Cols;
  const int T = build_tile_table(offsets, G, kTileRows, tl) * NT;
  const int64_t rtb = (int64_t)kTileRows * args.K;  // bytes of a tile's operand panel (fp8 codes)
  const int grid = gridDim.x;
  const int r = T % grid;
  const int half = (r > 0 && 2 * r <= grid && T > grid) ? r : 0;
  const int entries = T + half;
  const Shuffle sm = make_shuffle(shuffle, T - half), sh = make_shuffle(shuffle, half);
  for (int v = xcd_slot(blockIdx.x, grid); v < entries; v += grid) {
    if (v < T - half) {
      const TileCoord c = tile_coord(shuffled(sm, v), G, NT, kTileRows, xcd_slots, rtb, tl);
      if (tl.seg_rows[c.g] <= kTileRows / 2)
        mx_gemm_tile<kTileRows / 2>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
      else
        mx_gemm_tile<kTileRows>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
    } else {
      const int j = v - (T - half);
      const TileCoord c = tile_coord(T - half + shuffled(sh, j / 2), G, NT, kTileRows, xcd_slots, rtb, tl);
      const int m0 = c.m0 + (j & 1) * (kTileRows / 2);
      if (m0 < tl.seg_rows[c.g]) mx_gemm_tile<kTileRows / 2>(args, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], m0, c.nt, lds);
    }
  }
}

// MXFP8 quantisation of rows x cols values (bf16 or f32; cols a multiple of
// 128), one thread per scale byte, in storage order: codes [rows, cols];
// scale bytes in groups of 32 rows (rows padded to a multiple of 32; the
// padding's bytes are 0), for each 128-column quad the 4 bytes of each row.
__global__ __launch_bounds__(256) void mx_quantize_kernel(const void* __restrict__ src, int src_bf16, int64_t rows,
                                                          int cols, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t nblk = (rows + 31) / 32 * 32 * (cols / 32);
  for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < nblk; s += (int64_t)gridDim.x * blockDim.x) {
    const int64_t grp = s / cols;
    const int in = (int)(s - grp * cols);  // byte inside the group's cols bytes
    const int64_t r = grp * 32 + ((in & 127) >> 2);
    const int j = (in >> 7) * 4 + (in & 3);  // block of row r
    if (r >= rows) {
      scales[s] = 0;
      continue;
    }
    const int64_t b = r * (cols / 32) + j;
    float v[32];
    if (src_bf16) {
      const bf16x8_t* s8 = reinterpret_cast<const bf16x8_t*>(src) + b * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t w = s8[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * i + j] = (float)w[j];
      }
    } else {
      const f32x4_t* s4 = reinterpret_cast<const f32x4_t*>(src) + b * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4_t w = s4[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = w[j];
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int X = mx_scale(amax);
    i32x4_t out[2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      out[i / 4][i % 4] = (int)e4m3_pack4(ldexpf(v[4 * i], -X), ldexpf(v[4 * i + 1], -X), ldexpf(v[4 * i + 2], -X),
                                          ldexpf(v[4 * i + 3], -X));
    *reinterpret_cast<i32x4_t*>(codes + b * 32) = out[0];
    *reinterpret_cast<i32x4_t*>(codes + b * 32 + 16) = out[1];
    scales[s] = (uint8_t)(X + 127);
  }
}

// Second pass of a split last round (layer 1): for every split tile, add
// the partial accumulators of its K ranges in increasing order (f32) and
// store Y.  Work item = (split tile, 16 token rows); 64 threads per token
// row, 4 columns each.
constexpr int kReduceRows = 16;

__global__ __launch_bounds__(256) void grouped_gemm_split_reduce(Bf16GemmArgs args, SplitWs split) {
  const int r = split.hdr[0], s = split.hdr[1];
  if (r == 0) return;
  const int N = args.N;
  const int items = r * (kTileRows / kReduceRows);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int jj = it / (kTileRows / kReduceRows);
    const int t0 = (it % (kTileRows / kReduceRows)) * kReduceRows;
    const int32_t* d = split.desc + 4 * jj;
    const int seg_start = d[0], seg_rows = d[1], m0 = d[2], nt = d[3];
    const float* base = split.part + (size_t)jj * s * kSplitPartFloats;
    const int c = threadIdx.x & 63;
    const int n = nt * kL1Cols + 4 * c;
    // the thread's 4 rows t0 + (tid / 64) + 4 i accumulate together, so 4
    // loads are in flight per range; each sum still runs over the ranges in
    // increasing order from zero (rows past the segment are read from the
    // partial buffer, which has all 256, and not stored)
    constexpr int RT = kReduceRows / 4;
    const int tq = t0 + (threadIdx.x >> 6);
    f32x4_t ys[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) ys[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < s; ++k) {
      const float* pk = base + (size_t)k * kSplitPartFloats + 4 * c;
#pragma unroll
      for (int i = 0; i < RT; ++i) ys[i] += *reinterpret_cast<const f32x4_t*>(pk + (size_t)(tq + 4 * i) * 256);
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int trow = m0 + tq + 4 * i;
      if (trow < seg_rows && n < N)
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(args.c) + (int64_t)(seg_start + trow) * N + n) = ys[i];
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
                                                               int G, uint32_t shuffle) {
  __shared__ float xs[kF32Rows][kF32BK + 1];
  __shared__ float ws[kF32Rows][kF32BK + 1];
  __shared__ TileLds tl;
  constexpr int cols = (LAYER == 0) ? kF32Rows / 2 : kF32Rows;
  const int NT = (N + cols - 1) / cols;
  const int total = build_tile_table(offsets, G, kF32Rows, tl) * NT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const Shuffle sm = make_shuffle(shuffle, total);
  for (int v = blockIdx.x; v < total; v += gridDim.x) {
    const TileCoord c = tile_coord(shuffled(sm, v), G, NT, kF32Rows, 1, 0, tl);
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

size_t gemm_split_ws_bytes() {
  const size_t units = (size_t)device_cu_count();
  return kSplitHdrBytes + units * kSplitPartFloats * sizeof(float);
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
  a.c_scale = nullptr;
  a.a_scale = nullptr;
  a.w_scale = nullptr;
  a.a_scale_bytes = a.w_scale_bytes = 0;
  const int grid = device_cu_count();
  const int xcd_slots = grid / kXcds > 0 ? grid / kXcds : 1;
  if (gp.rowmap) {
    a.M = gp.R;  // rows of the token-row buffer, read at their own positions
    if (gp.layer == 0)
      grouped_gemm_bf16_expert_kernel<0><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, xcd_slots, gp.shuffle);
    else
      grouped_gemm_bf16_expert_kernel<1><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, xcd_slots, gp.shuffle);
    return hipGetLastError();
  }
  SplitWs sp{nullptr, nullptr, nullptr};
  // layer 1 only; the header holds descriptors of up to 4096 split tiles (fewer than the grid)
  if (gp.layer == 1 && gp.ws && gp.ws_bytes >= gemm_split_ws_bytes() && grid <= 4096) {
    char* w = reinterpret_cast<char*>(gp.ws);
    sp.hdr = reinterpret_cast<int32_t*>(w);
    sp.desc = sp.hdr + 4;
    sp.part = reinterpret_cast<float*>(w + kSplitHdrBytes);
  }
  if (gp.layer == 0)
    grouped_gemm_bf16_kernel<0><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, xcd_slots, sp, gp.shuffle);
  else
    grouped_gemm_bf16_kernel<1><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, xcd_slots, sp, gp.shuffle);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !sp.hdr) return e;
  // up to 4 blocks per split tile's 16 items of 16 rows (r <= grid tiles);
  // blocks past the items exit at once
  grouped_gemm_split_reduce<<<4 * grid, 256, 0, s>>>(a, sp);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_mx(const GemmProblem& gp, hipStream_t s) {
  if (gp.R == 0) return hipSuccess;
  Bf16GemmArgs a;
  a.K = gp.K;
  a.N = gp.N;
  a.E = gp.E;
  a.s2f = nullptr;
  a.topk = 1;
  a.M = 0;
  a.c_scale = nullptr;
  a.a_scale = nullptr;
  a.w_scale = nullptr;
  a.a_scale_bytes = a.w_scale_bytes = 0;
  const int grid = device_cu_count();
  const int xcd_slots = grid / kXcds > 0 ? grid / kXcds : 1;
  if (gp.layer == 0) {
    // x_perm, W_gate, W_up bf16; Hact MXFP8: R*F codes, then the scales
    a.a = (const __bf16*)gp.a;
    a.w0 = (const __bf16*)gp.w0;
    a.w1 = (const __bf16*)gp.w1;
    a.c = gp.c;
    a.c_scale = reinterpret_cast<uint8_t*>(gp.c) + gp.R * gp.N;
    grouped_gemm_bf16_kernel<0, true><<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, xcd_slots, SplitWs{},
                                                                     gp.shuffle);
  } else {
    // Hact and W_down MXFP8 (codes, then scales); Y f32
    a.a = (const __bf16*)gp.a;
    a.a_scale = reinterpret_cast<const uint8_t*>(gp.a) + gp.R * gp.K;
    a.a_scale_bytes = (uint32_t)mx_scale_bytes(gp.R, gp.K);
    a.w0 = (const __bf16*)gp.w0;
    a.w_scale = reinterpret_cast<const uint8_t*>(gp.w0) + (int64_t)gp.E * gp.N * gp.K;
    a.w_scale_bytes = (uint32_t)mx_scale_bytes((int64_t)gp.E * gp.N, gp.K);
    a.w1 = nullptr;
    a.c = gp.c;
    grouped_gemm_mx_kernel<<<grid, kGemmThreads, 0, s>>>(a, gp.offsets, gp.G, xcd_slots, gp.shuffle);
  }
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* src, int src_bf16, int64_t rows, int cols, void* dst, hipStream_t s) {
  const int64_t nblk = mx_scale_bytes(rows, cols);
  if (nblk == 0) return hipSuccess;
  uint8_t* codes = reinterpret_cast<uint8_t*>(dst);
  const int64_t blocks = (nblk + 255) / 256;
  mx_quantize_kernel<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(src, src_bf16, rows, cols, codes,
                                                                                  codes + rows * (int64_t)cols);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_f32(const GemmProblem& gp, hipStream_t s) {
  if (gp.R == 0) return hipSuccess;
  const int grid = device_cu_count() * 2;
  if (gp.layer == 0)
    grouped_gemm_f32_kernel<0><<<grid, 256, 0, s>>>((const float*)gp.a, (const float*)gp.w0, (const float*)gp.w1,
                                                     (float*)gp.c, gp.K, gp.N, gp.E, gp.offsets, gp.G, gp.shuffle);
  else
    grouped_gemm_f32_kernel<1><<<grid, 256, 0, s>>>((const float*)gp.a, (const float*)gp.w0, nullptr,
                                                    (float*)gp.c, gp.K, gp.N, gp.E, gp.offsets, gp.G, gp.shuffle);
  return hipGetLastError();
}

}  // namespace moe

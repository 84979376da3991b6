// Tile queue of the grouped GEMM: segments (expert problems of different
// row counts) cut into uniform tiles and ordered for cache reuse.
//
// "Grouped GEMM 为什么适合 MoE" (why grouped GEMM suits MoE), sections
// "1. Tiling" (uneven experts become uniform tiles a scheduler hands out)
// and "3. L2 cache conflict 缓解" (tile order decides L2 reuse of expert
// weights).  The table is derived on the device from the offsets array, so
// no host round trip sits between the dispatch and the GEMM.
//
// Order: segment by segment; inside a segment, column groups of GN tiles,
// and inside a group the row tiles fastest.  A persistent workgroup walks
// virtual slots it*grid + v, and v is chosen so that the workgroups of one
// XCD (hardware ids w, w+8, ... are dispatched round-robin over the 8 XCDs)
// own a contiguous run of slots: concurrently running tiles on one XCD then
// share the expert's weight columns and token rows in that XCD's L2.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMaxTileSegs = 1024;
constexpr int kXcds = 8;

struct TileTable {
  int G;
  int NT;     // column tiles per segment
  int rows;   // row tile height
  int total;  // total tiles
};

// Fills LDS arrays (each sized kMaxTileSegs + 1): seg_start[g] (first row),
// seg_rows[g], tile_start[g] (exclusive prefix of tiles); returns the total.
// All threads of the block must call it.
__device__ inline int build_tile_table(const int32_t* __restrict__ offsets, int G, int NT, int rows,
                                       int* seg_start, int* seg_rows, int* tile_start, int* scratch) {
  const int nthr = blockDim.x;
  // per-thread serial prefix over a contiguous run of segments, then a scan of run totals
  const int per = (G + nthr - 1) / nthr;
  const int g0 = threadIdx.x * per;
  int run = 0;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    const int a = offsets[g], b = offsets[g + 1];
    seg_start[g] = a;
    seg_rows[g] = b - a;
    run += ((b - a + rows - 1) / rows) * NT;
  }
  scratch[threadIdx.x] = run;
  __syncthreads();
  for (int off = 1; off < nthr; off <<= 1) {
    const int v = (threadIdx.x >= (unsigned)off) ? scratch[threadIdx.x - off] : 0;
    __syncthreads();
    scratch[threadIdx.x] += v;
    __syncthreads();
  }
  int acc = scratch[threadIdx.x] - run;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    tile_start[g] = acc;
    acc += ((seg_rows[g] + rows - 1) / rows) * NT;
  }
  const int total = scratch[nthr - 1];
  if (threadIdx.x == 0) tile_start[G] = total;
  __syncthreads();
  return total;
}

struct TileCoord {
  int g;       // segment
  int m0;      // first row of the tile inside the segment
  int nt;      // column tile index
};

// Map a tile index to (segment, row tile, column tile).
__device__ inline TileCoord tile_coord(int v, int G, int NT, int rows, int group_cols, const int* seg_rows,
                                       const int* tile_start) {
  int lo = 0, hi = G - 1;  // last g with tile_start[g] <= v
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= v) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int l = v - tile_start[g];
  const int mt = (seg_rows[g] + rows - 1) / rows;
  int gn = group_cols / (mt > 0 ? mt : 1);
  if (gn < 1) gn = 1;
  const int span = mt * gn;
  const int grp = l / span, rem = l - grp * span;
  TileCoord c;
  c.g = g;
  c.m0 = (rem % mt) * rows;
  c.nt = grp * gn + rem / mt;
  return c;
}

// Virtual slot of this workgroup: the workgroups of one XCD get a contiguous run.
__device__ __forceinline__ int xcd_slot(int wg, int grid) {
  if (grid % kXcds != 0) return wg;
  const int per = grid / kXcds;
  return (wg % kXcds) * per + wg / kXcds;
}

}  // namespace moe

// Tile queue of the grouped GEMM: segments (expert problems of different
// row counts) cut into uniform tiles and ordered for cache reuse.
//
// "Grouped GEMM 为什么适合 MoE" (why grouped GEMM suits MoE), sections
// "1. Tiling" (uneven experts become uniform tiles a scheduler hands out)
// and "3. L2 cache conflict 缓解" (tile order decides L2 reuse of expert
// weights).  The table is derived on the device from the offsets array, so
// no host round trip sits between the dispatch and the GEMM.
//
// A segment of n rows has ceil(n / rows) row tiles ("M-tiles"); mt_start[g]
// is the exclusive prefix of the M-tile counts.  With NT column tiles, the
// tiles of segment g occupy [mt_start[g] * NT, mt_start[g+1] * NT) of the
// queue, row tiles fastest, in blocks of row tiles (tile_coord).  A
// persistent workgroup walks virtual slots
// it*grid + v, and v is chosen so that the workgroups of one XCD (hardware
// ids w, w+8, ... are dispatched round-robin over the 8 XCDs) own a
// contiguous run of slots: concurrently running tiles on one XCD then share
// the expert's weight columns and token rows in that XCD's L2.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMaxTileSegs = 1024;
constexpr int kXcds = 8;

struct TileLds {
  int seg_start[kMaxTileSegs + 1];
  int seg_rows[kMaxTileSegs + 1];
  int mt_start[kMaxTileSegs + 1];
  int scratch[256];
  int expert_rows[kMaxTileSegs / 2 + 1];  // rows of each expert over all source blocks (row-map tables)
};

// Fills seg_start, seg_rows and mt_start from offsets; returns the number of
// M-tiles.  All threads of the block (<= 256) must call it.
__device__ inline int build_tile_table(const int32_t* __restrict__ offsets, int G, int rows, TileLds& t) {
  const int nthr = blockDim.x;
  const int per = (G + nthr - 1) / nthr;
  const int g0 = threadIdx.x * per;
  int run = 0;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    const int a = offsets[g], b = offsets[g + 1];
    t.seg_start[g] = a;
    t.seg_rows[g] = b - a;
    run += (b - a + rows - 1) / rows;
  }
  t.scratch[threadIdx.x] = run;
  __syncthreads();
  for (int off = 1; off < nthr; off <<= 1) {
    const int v = (threadIdx.x >= (unsigned)off) ? t.scratch[threadIdx.x - off] : 0;
    __syncthreads();
    t.scratch[threadIdx.x] += v;
    __syncthreads();
  }
  int acc = t.scratch[threadIdx.x] - run;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    t.mt_start[g] = acc;
    acc += (t.seg_rows[g] + rows - 1) / rows;
  }
  const int total = t.scratch[nthr - 1];
  if (threadIdx.x == 0) t.mt_start[G] = total;
  __syncthreads();
  return total;
}

// The table of a grouped GEMM whose segments are S = G / EL source blocks of
// EL experts each (segment g = s EL + e): each expert's rows, over all its
// source blocks, form one combined segment, so a tile of 256 rows can take
// rows of several small segments of the same expert and every weight panel
// serves full tiles.  Fills seg_start and seg_rows of the G segments,
// expert_rows[e] and mt_start[e] (prefix of the experts' M-tile counts);
// returns the number of M-tiles.  All threads of the block (<= 256) call it.
__device__ inline int build_expert_tile_table(const int32_t* __restrict__ offsets, int G, int EL, int rows,
                                              TileLds& t) {
  const int nthr = blockDim.x;
  for (int g = threadIdx.x; g < G; g += nthr) {
    t.seg_start[g] = offsets[g];
    t.seg_rows[g] = offsets[g + 1] - offsets[g];
  }
  __syncthreads();
  const int S = G / EL;
  const int per = (EL + nthr - 1) / nthr;
  const int e0 = threadIdx.x * per;
  int run = 0;
  for (int e = e0; e < e0 + per && e < EL; ++e) {
    int n = 0;
    for (int s = 0; s < S; ++s) n += t.seg_rows[s * EL + e];
    t.expert_rows[e] = n;
    run += (n + rows - 1) / rows;
  }
  t.scratch[threadIdx.x] = run;
  __syncthreads();
  for (int off = 1; off < nthr; off <<= 1) {
    const int v = (threadIdx.x >= (unsigned)off) ? t.scratch[threadIdx.x - off] : 0;
    __syncthreads();
    t.scratch[threadIdx.x] += v;
    __syncthreads();
  }
  int acc = t.scratch[threadIdx.x] - run;
  for (int e = e0; e < e0 + per && e < EL; ++e) {
    t.mt_start[e] = acc;
    acc += (t.expert_rows[e] + rows - 1) / rows;
  }
  const int total = t.scratch[nthr - 1];
  if (threadIdx.x == 0) t.mt_start[EL] = total;
  __syncthreads();
  return total;
}

// Sorted row of row m0 + i (i < n) of expert e's combined segment, -1 past
// its rows: the source blocks' segments in order.
__device__ inline int expert_row(const TileLds& t, int e, int EL, int S, int m0, int i) {
  int r = m0 + i;
  if (r >= t.expert_rows[e]) return -1;
  for (int s = 0; s < S; ++s) {
    const int n = t.seg_rows[s * EL + e];
    if (r < n) return t.seg_start[s * EL + e] + r;
    r -= n;
  }
  return -1;
}

// Last segment g with mt_start[g] * mult <= v (v below the total).
__device__ inline int find_segment(int v, int G, int mult, const int* mt_start) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mt_start[mid] * mult <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct TileCoord {
  int g;   // segment
  int m0;  // first row of the tile inside the segment
  int nt;  // column tile index (relative to the column range the queue covers)
  int mt;  // global M-tile index
};

// What the last-level cache (256 MB on MI355X, shared by the XCDs) keeps
// while a segment's tiles go by: its token rows up to kResidentRowBytes,
// its weight panels up to kResidentWeightBytes (the weights are read in a
// second pass over them, the token rows over and over).
constexpr int64_t kResidentRowBytes = 64ll << 20;
constexpr int64_t kResidentWeightBytes = 128ll << 20;

// Tile v of a queue over NT column tiles (per segment mt_g * NT tiles).
// panel_bytes is the bytes of one tile's operand panel over the whole
// reduction (tokens of a row tile, weights of a column tile: both 256 rows);
// xcd_slots is the number of tiles one XCD runs at once (its workgroups).
// Inside a segment (or a row block of it, below) the order is column-major
// with the row tiles fastest: consecutive entries are the row tiles of one
// weight column tile, then of the next column tile, so the tiles an XCD runs
// at once (a contiguous run of the order, see xcd_slot) share a few weight
// panels and a few token panels in its L2, and each weight panel is read
// once while the segment's token rows are re-read from the cache.  A
// segment of more than xcd_slots / 4 row tiles whose token rows are too big
// for the cache, or whose weight panels are small enough to be read twice
// from it, is cut into nb = ceil(mt / (xcd_slots / 4)) blocks of row tiles
// of nearly equal height, each ordered as a segment of its own (so an XCD's
// run spans about 8 row tiles x 4 column tiles instead of one column of
// every row tile).  Block b holds rows [b mt / nb, (b + 1) mt / nb), i.e.
// queue entries [row0 NT, row1 NT).
__device__ inline TileCoord tile_coord(int v, int G, int NT, int rows, int xcd_slots, int64_t panel_bytes,
                                       const TileLds& t) {
  const int g = find_segment(v, G, NT, t.mt_start);
  const int l = v - t.mt_start[g] * NT;
  const int mt = t.mt_start[g + 1] - t.mt_start[g];
  const int rbmax = xcd_slots / 4 > 0 ? xcd_slots / 4 : 1;
  const bool block = panel_bytes > 0 && mt > rbmax &&
                     ((int64_t)mt * panel_bytes > kResidentRowBytes || (int64_t)NT * panel_bytes <= kResidentWeightBytes);
  int r0 = 0, rb = mt, lb = l;
  if (block) {
    const int nb = (mt + rbmax - 1) / rbmax;
    auto row_of = [&](int bb) { return (int)(((int64_t)bb * mt) / nb); };  // first row of block bb
    const int r = l / NT;  // a row of l's block
    int b = (int)(((int64_t)r * nb) / mt);
    if (b > nb - 1) b = nb - 1;
    if (row_of(b + 1) <= r) ++b;
    r0 = row_of(b);
    rb = row_of(b + 1) - r0;
    lb = l - r0 * NT;
  }
  TileCoord c;
  c.g = g;
  const int mi = r0 + lb % rb;
  c.m0 = mi * rows;
  c.nt = lb / rb;
  c.mt = t.mt_start[g] + mi;
  return c;
}

// Seeded reordering of n interchangeable items (the MOE_DEBUG_SHUFFLE
// check): i -> (a i + b) mod n with a coprime to n, a bijection of [0, n).
// Seed 0 gives the identity.  Every output element is computed by one item
// in a fixed order of its own, so a reordering must not change any bit.
struct Shuffle {
  uint32_t a, b, n;
};

__device__ inline Shuffle make_shuffle(uint32_t seed, int n) {
  Shuffle s{1u, 0u, n > 1 ? (uint32_t)n : 1u};
  if (seed == 0 || n <= 1) return s;
  auto gcd = [](uint32_t x, uint32_t y) {
    while (y) {
      const uint32_t t = x % y;
      x = y;
      y = t;
    }
    return x;
  };
  uint32_t a = (seed * 2654435761u) % s.n;
  if (a == 0) a = 1;
  while (gcd(a, s.n) != 1) a = a + 1 < s.n ? a + 1 : 1;
  s.a = a;
  s.b = ((seed ^ (seed >> 16)) * 40503u) % s.n;
  return s;
}

__device__ __forceinline__ int shuffled(const Shuffle& s, int i) {
  return s.a == 1u && s.b == 0u ? i : (int)(((uint64_t)s.a * (uint32_t)i + s.b) % s.n);
}

// Virtual slot of workgroup `wg` among `n` workgroups: the workgroups of one
// XCD get a contiguous run of slots.
__device__ __forceinline__ int xcd_slot(int wg, int n) {
  if (n % kXcds != 0) return wg;
  const int per = n / kXcds;
  return (wg % kXcds) * per + wg / kXcds;
}

}  // namespace moe

// Counts, offsets, stable permutation and the dispatch copy.
//
// PTO MoE article (seven serial stages: local reorder by expert; the
// count-as-flag paragraph: per-expert row counts) and COMET paper review
// §4.1.2 (Layer0: order tokens by source first).  Pair f = t*k + j goes to
// segment g = src_block[t] * EL + (topk_idx[t, j] - base) when its expert is
// one of the EL held here, and is dropped otherwise; the sorted order lists
// the segments in turn and, inside a segment, the pairs by increasing f.
// Dropped pairs are ranked as one more segment after the G reported ones,
// so they take the sorted positions past the kept pairs; those positions
// and the dropped pairs' flat_to_sorted entries are written as -1.
//
// No atomic operation decides an order, so every output is bit-exact and
// independent of scheduling:
//   seg_count  one block per chunk of pairs: LDS histogram over the G
//              segments (atomics only add counts, which commute).
//   seg_scan   one block: per segment, exclusive prefix over the chunks;
//              counts; exclusive prefix over segments = offsets; the
//              start of every (chunk, segment) run.
//   seg_rank   one block per chunk, walking it 256 pairs at a time in flat
//              order: inside a wave, lanes with equal keys find each other
//              with one ballot per key bit, and the rank among them is a
//              popcount of the lower lanes; waves are ordered through a small
//              per-wave count table in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxSegments = 1024;

// Segment of pair f; G (one past the reported segments) if dropped.
__device__ __forceinline__ int seg_of(const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ src_block,
                                      int ebase, int EL, int G, int k, int64_t f) {
  const int s = src_block ? src_block[f / k] : 0;
  const unsigned e = (unsigned)(topk_idx[f] - ebase);
  return e < (unsigned)EL ? s * EL + (int)e : G;
}

// Histograms over the Gi ranked segments (Gi = G, or G + 1 with dropped pairs).
__global__ __launch_bounds__(kPermThreads) void seg_count_kernel(const int32_t* __restrict__ topk_idx,
                                                                 const int32_t* __restrict__ src_block, int ebase,
                                                                 int EL, int k, int64_t R, int G, int Gi, int chunk,
                                                                 int32_t* __restrict__ block_hist) {
  __shared__ int hist[kMaxSegments];
  for (int g = threadIdx.x; g < Gi; g += kPermThreads) hist[g] = 0;
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  const int64_t end = (begin + chunk < R) ? begin + chunk : R;
  for (int64_t f = begin + threadIdx.x; f < end; f += kPermThreads)
    atomicAdd(&hist[seg_of(topk_idx, src_block, ebase, EL, G, k, f)], 1);
  __syncthreads();
  for (int g = threadIdx.x; g < Gi; g += kPermThreads) block_hist[(int64_t)blockIdx.x * Gi + g] = hist[g];
}

// Column-wise exclusive scan of block_hist [blocks][G] (in place), the
// per-segment totals (counts) and their exclusive scan (offsets).  Thread
// layout: P = 1024 / G' threads per segment (G' = G rounded up to a power of
// two), each owning a contiguous slice of the blocks, so every thread issues
// independent loads and the chain of dependent adds stays short.  Here G is
// the number of ranked segments; the first Gr are reported: counts[0..Gr-1]
// and offsets[0..Gr], where offsets[Gr] is the start of the dropped pairs'
// segment when G > Gr, else R.
__global__ __launch_bounds__(kMaxSegments) void seg_scan_kernel(int G, int Gr, int blocks, int64_t R,
                                                                int32_t* __restrict__ block_hist,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int part[kMaxSegments];
  __shared__ int s[kMaxSegments];
  __shared__ int tot[kMaxSegments];
  int gp = 1;
  while (gp < G) gp <<= 1;
  // slices per segment: as many as fit, but no more than there are blocks
  // (the prefix over slices below is serial in P)
  int P = kMaxSegments / gp;
  if (P > blocks) P = blocks > 0 ? blocks : 1;
  const int g = threadIdx.x % gp, p = threadIdx.x / gp;
  const bool active = p < P;
  const int L = (blocks + P - 1) / P;
  const int b0 = p * L, b1 = min(blocks, b0 + L);
  int sum = 0;
  if (active && g < G)
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += block_hist[(int64_t)b * G + g];
  if (active) part[threadIdx.x] = sum;
  __syncthreads();
  // exclusive prefix over the P slices of each segment, and the segment total
  if (threadIdx.x < gp) {
    int run = 0;
    for (int q = 0; q < P; ++q) {
      const int v = part[q * gp + threadIdx.x];
      part[q * gp + threadIdx.x] = run;
      run += v;
    }
    s[threadIdx.x] = (threadIdx.x < G) ? run : 0;
  }
  __syncthreads();
  const int total = (threadIdx.x < gp) ? s[threadIdx.x] : 0;
  if (threadIdx.x < gp) tot[threadIdx.x] = total;
  if (threadIdx.x < Gr) counts[threadIdx.x] = total;
  // exclusive scan of the totals over segments
  for (int off = 1; off < gp; off <<= 1) {
    const int v = (threadIdx.x < gp && threadIdx.x >= (unsigned)off) ? s[threadIdx.x - off] : 0;
    __syncthreads();
    if (threadIdx.x < gp) s[threadIdx.x] += v;
    __syncthreads();
  }
  if (threadIdx.x < G && threadIdx.x <= Gr) offsets[threadIdx.x] = s[threadIdx.x] - total;
  if (G == Gr && threadIdx.x == 0) offsets[Gr] = (int)R;
  __syncthreads();
  // block_hist[b][g] <- offsets[g] + pairs of segment g in blocks before b
  if (active && g < G) {
    int run = s[g] - tot[g] + part[threadIdx.x];  // offsets[g] + blocks before this slice
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      const int v = block_hist[(int64_t)b * G + g];
      block_hist[(int64_t)b * G + g] = run;
      run += v;
    }
  }
}

// Ranks over the Gi ranked segments; a dropped pair (segment G) writes -1.
__global__ __launch_bounds__(kPermThreads) void seg_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                                const int32_t* __restrict__ src_block, int ebase,
                                                                int EL, int k, int64_t R, int G, int Gi, int chunk,
                                                                int nbits,
                                                                const int32_t* __restrict__ block_base,
                                                                int32_t* __restrict__ sorted_to_flat,
                                                                int32_t* __restrict__ flat_to_sorted) {
  __shared__ int running[kMaxSegments];
  __shared__ int wcnt[kPermWaves][kMaxSegments];
  const int tid = threadIdx.x, w = tid / kWave;
  for (int g = tid; g < Gi; g += kPermThreads) {
    running[g] = block_base[(int64_t)blockIdx.x * Gi + g];
#pragma unroll
    for (int q = 0; q < kPermWaves; ++q) wcnt[q][g] = 0;
  }
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  const int64_t end = (begin + chunk < R) ? begin + chunk : R;
  const uint64_t below = lanemask_lt();
  for (int64_t base = begin; base < end; base += kPermThreads) {
    const int64_t f = base + tid;
    const bool valid = f < end;
    const int g = valid ? seg_of(topk_idx, src_block, ebase, EL, G, k, f) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const int bit = (g >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank = __popcll(peers & below);
    const int group = __popcll(peers);
    if (valid && rank == 0) wcnt[w][g] = group;
    __syncthreads();
    if (valid) {
      int pos = running[g] + rank;
      for (int q = 0; q < w; ++q) pos += wcnt[q][g];
      const bool kept = g < G;
      sorted_to_flat[pos] = kept ? (int32_t)f : -1;
      flat_to_sorted[f] = kept ? pos : -1;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&running[g], group);
      wcnt[w][g] = 0;
    }
    __syncthreads();
  }
}

PermutePlan permute_plan(int64_t M, int k, int S, int E, int base, int EL) {
  PermutePlan pl;
  pl.R = M * k;
  pl.EL = EL > 0 ? EL : E;
  pl.base = EL > 0 ? base : 0;
  pl.G = S * pl.EL;
  pl.Gi = pl.G + (pl.EL < E ? 1 : 0);
  // small chunks: many blocks rank in parallel (the ranking of one chunk is
  // sequential in steps of 256 pairs)
  int64_t chunk = 512;
  const int64_t want = (pl.R + 1023) / 1024;  // at most 1024 chunks
  if (want > chunk) chunk = ((want + kPermThreads - 1) / kPermThreads) * kPermThreads;
  pl.chunk = (int)chunk;
  pl.blocks = (int)((pl.R + chunk - 1) / chunk);
  return pl;
}

size_t permute_ws_bytes(const PermutePlan& pl) { return (size_t)(pl.blocks > 0 ? pl.blocks : 1) * pl.Gi * 4; }

hipError_t launch_permute(const PermutePlan& pl, const int32_t* topk_idx, const int32_t* src_block, int k,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                          int32_t* ws, hipStream_t s) {
  int nbits = 1;
  while ((1 << nbits) < pl.Gi) ++nbits;
  if (pl.blocks > 0)
    seg_count_kernel<<<pl.blocks, kPermThreads, 0, s>>>(topk_idx, src_block, pl.base, pl.EL, k, pl.R, pl.G, pl.Gi,
                                                        pl.chunk, ws);
  seg_scan_kernel<<<1, kMaxSegments, 0, s>>>(pl.Gi, pl.G, pl.blocks, pl.R, ws, counts, offsets);
  if (pl.blocks > 0)
    seg_rank_kernel<<<pl.blocks, kPermThreads, 0, s>>>(topk_idx, src_block, pl.base, pl.EL, k, pl.R, pl.G, pl.Gi,
                                                       pl.chunk, nbits, ws, sorted_to_flat, flat_to_sorted);
  return hipGetLastError();
}

// ------------------------------------------------------------ dispatch ---
// Each token row is read once and written to its k sorted positions,
// 16 bytes per lane; a block walks whole rows (two at a time, so each lane
// has several loads in flight) and the writes of one row are contiguous.
// X_perm is written with ordinary stores (measured on MI355X: 33.7 us for
// Mixtral's 201 MB against 39.7 us with non-temporal stores).
constexpr int kCopyThreads = 256;
constexpr int kCopyRows = 2;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void dispatch_copy_kernel(const u32x4_t* __restrict__ x, int64_t M,
                                                                     int C, int k, const int32_t* __restrict__ f2s,
                                                                     u32x4_t* __restrict__ xp) {
  for (int64_t t0 = (int64_t)blockIdx.x * kCopyRows; t0 < M; t0 += (int64_t)gridDim.x * kCopyRows) {
    const int nr = (M - t0) < kCopyRows ? (int)(M - t0) : kCopyRows;
    // a token none of whose pairs is held here is not read at all
    bool need[kCopyRows];
#pragma unroll
    for (int r = 0; r < kCopyRows; ++r) {
      need[r] = false;
      if (r < nr)
        for (int j = 0; j < k; ++j) need[r] |= f2s[(t0 + r) * k + j] >= 0;
    }
    for (int c0 = threadIdx.x; c0 < C; c0 += kCopyThreads * 2) {
      u32x4_t v[kCopyRows][2];
#pragma unroll
      for (int r = 0; r < kCopyRows; ++r)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = c0 + u * kCopyThreads;
          if (need[r] && c < C) v[r][u] = x[(t0 + r) * C + c];
        }
#pragma unroll
      for (int r = 0; r < kCopyRows; ++r) {
        if (r >= nr || !need[r]) continue;
        for (int j = 0; j < k; ++j) {
          const int32_t row = f2s[(t0 + r) * k + j];
          if (row < 0) continue;  // pair of an expert not held here
          u32x4_t* d = xp + (int64_t)row * C;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int c = c0 + u * kCopyThreads;
            if (c < C) d[c] = v[r][u];
          }
        }
      }
    }
  }
}

hipError_t launch_dispatch_copy(const void* x, int64_t M, int64_t row_bytes, int k, const int32_t* flat_to_sorted,
                                void* x_perm, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int C = (int)(row_bytes / 16);
  const int64_t pairs = (M + kCopyRows - 1) / kCopyRows;
  const int64_t grid = pairs < 16384 ? pairs : 16384;
  dispatch_copy_kernel<<<(unsigned)grid, kCopyThreads, 0, s>>>((const u32x4_t*)x, M, C, k, flat_to_sorted,
                                                               (u32x4_t*)x_perm);
  return hipGetLastError();
}

}  // namespace moe

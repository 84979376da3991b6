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
// independent of scheduling.  The tokens are cut into chunks of Tc tokens
// (Tc k pairs), and each chunk into workgroups of Ts tokens:
//   seg_count       one block per chunk: LDS histogram over the segments
//                   (atomics only add counts, which commute).
//   dispatch_kernel one workgroup per Ts tokens.  It first issues the loads
//                   of its first token rows, then derives its chunk's
//                   segment bases from all chunks' histograms (segment
//                   totals, their exclusive prefix = offsets, plus the
//                   counts of earlier chunks), ranks the pairs from its
//                   chunk's start to its last token in steps of 256 (lanes
//                   with equal keys find each other with one ballot per key
//                   bit, the rank among them is a popcount of the lower
//                   lanes, waves are ordered through a per-wave count table
//                   in LDS), writes the permutation entries of its own
//                   pairs, and copies its token rows to their sorted
//                   positions (each row read once, written k times).
// When the histograms are too many for every workgroup to sum them
// (chunks x segments past kMaxSummed), one more kernel, seg_scan, turns
// them into the chunks' bases first and dispatch_kernel reads those.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxSegments = 1024;

// Segment of pair f; G (one past the reported segments) if dropped.  An
// expert id or source block out of range (a caller's error, which
// MOE_DEBUG_VALIDATE reports) also gives G, so the pair is ranked in the
// dropped segment or not at all, and no index leaves its array.
__device__ __forceinline__ int seg_of(const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ src_block,
                                      int ebase, int EL, int G, int k, int64_t f) {
  const unsigned s = src_block ? (unsigned)src_block[f / k] : 0u;
  const unsigned e = (unsigned)(topk_idx[f] - ebase);
  return (e < (unsigned)EL && s < (unsigned)(G / EL)) ? (int)s * EL + (int)e : G;
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
  for (int64_t f = begin + threadIdx.x; f < end; f += kPermThreads) {
    const int g = seg_of(topk_idx, src_block, ebase, EL, G, k, f);
    if (g < Gi) atomicAdd(&hist[g], 1);
  }
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
  // every pair is ranked (R in total) unless an expert id was out of range
  if (G == Gr && threadIdx.x == 0) offsets[Gr] = s[G - 1];
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

// ------------------------------------------------------------ dispatch ---
constexpr int kMaxOwnPairs = 256;      // pairs of one dispatch workgroup: Ts k <= 256
constexpr int kMaxSummed = 16384;      // chunks x segments one workgroup sums itself
constexpr int kMaxChunkPairs = 2048;   // pairs a workgroup ranks at most (8 steps of 256)
constexpr int kCopyRows = 2;           // token rows per copy step (loads in flight per lane)
#ifndef MOE_DISPATCH_WGS
#define MOE_DISPATCH_WGS 1024
#endif
constexpr int64_t kDispatchWgs = MOE_DISPATCH_WGS;  // workgroups the plan aims for
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct DispatchArgs {
  const int32_t* topk_idx;
  const int32_t* src_block;
  int ebase, EL, k, G, Gi, nbits;
  int64_t M;
  int Tc, Ts, chunks;
  const int32_t* hist;  // [chunks][Gi]: histograms, or (scanned) the chunks' bases
  int32_t* counts;
  int32_t* offsets;
  int32_t* s2f;
  int32_t* f2s;
  const u32x4_t* x;  // token rows, C 16-byte units each; null: no copy
  u32x4_t* xp;
  int C;
};

// Exclusive prefix sum of v[0..n) in place (n <= kMaxSegments), done by
// the first wave (lane l owns up to 16 consecutive entries; one shuffle scan
// over the lanes), so the block waits at one barrier only; all threads call
// it and get the total.  word: one int of LDS.
__device__ int block_exclusive_scan(int* v, int n, int* word) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (n + kWave - 1) / kWave;
    const int i0 = lane * per, i1 = i0 + per < n ? i0 + per : n;
    int run = 0;
    for (int i = i0; i < i1; ++i) run += v[i];
    int inc = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    int acc = inc - run;
    for (int i = i0; i < i1; ++i) {
      const int c = v[i];
      v[i] = acc;
      acc += c;
    }
    if (lane == kWave - 1) *word = inc;
  }
  __syncthreads();
  return *word;
}

// UPR: 16-byte units of a token row per thread (rows of at most 256 UPR
// units), so a batch of 16 / UPR rows sits in 16 registers of 16 bytes per
// thread; 0: rows of any width, copied two rows at a time.
template <bool SCANNED, int UPR>
__global__ __launch_bounds__(kPermThreads) void dispatch_kernel(DispatchArgs a) {
  __shared__ int base[kMaxSegments];              // next sorted position of each segment
  __shared__ int tot[kMaxSegments];               // segment totals, then their prefix
  __shared__ int wcnt[kPermWaves][kMaxSegments];  // pairs per wave and segment in the current step
  __shared__ int pos_lds[kMaxOwnPairs];           // sorted position of each own pair (-1: none)
  __shared__ int word;
  const int tid = threadIdx.x, w = tid / kWave;
  const int k = a.k, Gi = a.Gi;
  const int64_t t0 = (int64_t)blockIdx.x * a.Ts;
  const int64_t t1 = t0 + a.Ts < a.M ? t0 + a.Ts : a.M;
  const int c = (int)(t0 / a.Tc);
  const int64_t fbeg = (int64_t)c * a.Tc * k;  // first pair of the chunk
  const int64_t own0 = t0 * k, own1 = t1 * k;  // own pairs

  // (1) the first batch of token rows is loaded before the bookkeeping, so
  // the loads are in flight meanwhile (a token none of whose experts is held
  // here is not read)
  constexpr int RB = UPR > 0 ? 16 / UPR : kCopyRows;  // rows per batch
  constexpr int UU = UPR > 0 ? UPR : 2;               // units per thread per row and step
  u32x4_t v[RB][UU];
  const bool copy = a.x != nullptr;
  if (copy) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      bool held = false;
      if (t0 + r < t1)
        for (int j = 0; j < k; ++j) held |= (unsigned)(a.topk_idx[(t0 + r) * k + j] - a.ebase) < (unsigned)a.EL;
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const int cc = tid + u * kPermThreads;
        if (held && cc < a.C) v[r][u] = a.x[(t0 + r) * a.C + cc];
      }
    }
  }

  // (2) bases of this chunk's segments
  for (int g = tid; g < Gi; g += kPermThreads) {
#pragma unroll
    for (int q = 0; q < kPermWaves; ++q) wcnt[q][g] = 0;
    if (SCANNED) base[g] = a.hist[(int64_t)c * Gi + g];
    else base[g] = tot[g] = 0;
  }
  __syncthreads();
  if (!SCANNED) {
    // per segment, the sum of its counts over all chunks (tot) and over the
    // chunks before this one (base): with at most 256 segments, P threads
    // per segment each sum a slice of the chunks (independent loads, all in
    // flight), then the P partial sums are added; with more, one thread per
    // segment walks every chunk
    int gp = 1;
    while (gp < Gi) gp <<= 1;
    if (gp <= kPermThreads) {
      const int P = kPermThreads / gp, g = tid % gp, q = tid / gp;
      const int L = (a.chunks + P - 1) / P;
      const int b0 = q * L, b1 = b0 + L < a.chunks ? b0 + L : a.chunks;
      int sb = 0, sa = 0;
      if (g < Gi) {
#pragma unroll 8
        for (int b = b0; b < b1; ++b) {
          const int v = a.hist[(int64_t)b * Gi + g];
          if (b < c) sb += v;
          else sa += v;
        }
      }
      wcnt[0][tid] = sb;
      wcnt[1][tid] = sa;
      __syncthreads();
      if (q == 0 && g < Gi) {
        int before = 0, after = 0;
        for (int r = 0; r < P; ++r) {
          before += wcnt[0][r * gp + g];
          after += wcnt[1][r * gp + g];
        }
        base[g] = before;
        tot[g] = before + after;
      }
      __syncthreads();
      // the two rows of partial sums back to the zeros the ranking starts from
      wcnt[0][tid] = 0;
      wcnt[1][tid] = 0;
    } else {
      for (int g = tid; g < Gi; g += kPermThreads) {
        int sb = 0, sa = 0;
#pragma unroll 8
        for (int b = 0; b < a.chunks; ++b) {
          const int v = a.hist[(int64_t)b * Gi + g];
          if (b < c) sb += v;
          else sa += v;
        }
        base[g] = sb;
        tot[g] = sb + sa;
      }
    }
    __syncthreads();
    if (blockIdx.x == 0)
      for (int g = tid; g < a.G; g += kPermThreads) a.counts[g] = tot[g];
    __syncthreads();
    const int ranked = block_exclusive_scan(tot, Gi, &word);  // tot = offsets
    for (int g = tid; g < Gi; g += kPermThreads) base[g] += tot[g];
    if (blockIdx.x == 0) {
      for (int g = tid; g < a.G; g += kPermThreads) a.offsets[g] = tot[g];
      // the kept pairs end where the dropped pairs' segment starts, or with the last ranked pair
      if (tid == 0) a.offsets[a.G] = a.G < Gi ? tot[a.G] : ranked;
    }
    __syncthreads();
  }

  // (3) ranks from the chunk's first pair to the last own pair
  const uint64_t below = lanemask_lt();
  for (int64_t sb = fbeg; sb < own1; sb += kPermThreads) {
    const int64_t f = sb + tid;
    const bool inr = f < own1;
    const int gf = inr ? seg_of(a.topk_idx, a.src_block, a.ebase, a.EL, a.G, k, f) : Gi;
    const bool valid = gf < Gi;  // an invalid expert id of a plain layer gets no position
    const int g = valid ? gf : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < a.nbits; ++b) {
      const int bit = (g >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank = __popcll(peers & below);
    const int group = __popcll(peers);
    if (valid && rank == 0) wcnt[w][g] = group;
    __syncthreads();
    if (inr && f >= own0) {
      int pos = -1;
      if (valid) {
        pos = base[g] + rank;
        for (int q = 0; q < w; ++q) pos += wcnt[q][g];
        a.s2f[pos] = g < a.G ? (int32_t)f : -1;
        if (g >= a.G) pos = -1;  // a pair of an expert not held here
      }
      a.f2s[f] = pos;
      pos_lds[f - own0] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&base[g], group);
      wcnt[w][g] = 0;
    }
    __syncthreads();
  }
  if (!copy) return;

  // (4) the copy: each row read once and written to its kept positions
  auto needed = [&](int64_t t) {
    bool nd = false;
    for (int j = 0; j < k; ++j) nd |= pos_lds[(t - t0) * k + j] >= 0;
    return nd;
  };
  if constexpr (UPR > 0) {
    for (int64_t tb = t0; tb < t1; tb += RB) {
      if (tb != t0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const bool nd = tb + r < t1 && needed(tb + r);
#pragma unroll
          for (int u = 0; u < UU; ++u) {
            const int cc = tid + u * kPermThreads;
            if (nd && cc < a.C) v[r][u] = a.x[(tb + r) * a.C + cc];
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (tb + r >= t1) continue;
        for (int j = 0; j < k; ++j) {
          const int row = pos_lds[(tb + r - t0) * k + j];
          if (row < 0) continue;
          u32x4_t* d = a.xp + (int64_t)row * a.C;
#pragma unroll
          for (int u = 0; u < UU; ++u) {
            const int cc = tid + u * kPermThreads;
            if (cc < a.C) d[cc] = v[r][u];
          }
        }
      }
    }
  } else {
    for (int64_t tr = t0; tr < t1; tr += kCopyRows) {
      const int nr = (t1 - tr) < kCopyRows ? (int)(t1 - tr) : kCopyRows;
      bool need[kCopyRows];
#pragma unroll
      for (int r = 0; r < kCopyRows; ++r) need[r] = r < nr && needed(tr + r);
      for (int c0 = tid; c0 < a.C; c0 += kPermThreads * 2) {
        if (tr != t0 || c0 != tid) {
#pragma unroll
          for (int r = 0; r < kCopyRows; ++r)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int cc = c0 + u * kPermThreads;
              if (need[r] && cc < a.C) v[r][u] = a.x[(tr + r) * a.C + cc];
            }
        }
#pragma unroll
        for (int r = 0; r < kCopyRows; ++r) {
          if (!need[r]) continue;
          for (int j = 0; j < k; ++j) {
            const int row = pos_lds[(tr - t0 + r) * k + j];
            if (row < 0) continue;
            u32x4_t* d = a.xp + (int64_t)row * a.C;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int cc = c0 + u * kPermThreads;
              if (cc < a.C) d[cc] = v[r][u];
            }
          }
        }
      }
    }
  }
}

// Tokens per chunk Tc (a multiple of 16) and per workgroup Ts (a power of
// two up to 16, so Ts k <= kMaxOwnPairs for k <= 16).  Chunks of
// about 512 pairs; at most 1024 of them; when every workgroup can sum the
// histograms itself (chunks x segments <= kMaxSummed with chunks of at most
// kMaxChunkPairs pairs) the chunks grow to make that so.
PermutePlan permute_plan(int64_t M, int k, int S, int E, int base, int EL) {
  PermutePlan pl;
  pl.M = M;
  pl.k = k;
  pl.R = M * k;
  pl.EL = EL > 0 ? EL : E;
  pl.base = EL > 0 ? base : 0;
  pl.G = S * pl.EL;
  pl.Gi = pl.G + (pl.EL < E ? 1 : 0);
  // about 1024 workgroups (4 per CU on 256 CUs, all resident, so every
  // CU has enough row loads in flight), 2 to 16 tokens each
  pl.Ts = 2;
  while (pl.Ts < 16 && (int64_t)pl.Ts * kDispatchWgs < M) pl.Ts *= 2;
  // chunks are whole multiples of 16 tokens, so of any Ts
  auto round_up = [&](int64_t t) { return ((t + 15) / 16) * 16; };
  int64_t Tc = round_up((512 + k - 1) / k);
  const int64_t at_most = round_up((M + 1023) / 1024);  // at most 1024 chunks
  if (at_most > Tc) Tc = at_most;
  const int64_t summed = round_up((M * pl.Gi + kMaxSummed - 1) / kMaxSummed);
  pl.scanned = 1;
  if (summed * k <= kMaxChunkPairs) {
    if (summed > Tc) Tc = summed;
    pl.scanned = Tc * k > kMaxChunkPairs;
  }
  pl.Tc = (int)Tc;
  pl.blocks = (int)((M + Tc - 1) / Tc);
  pl.wgs = (M + pl.Ts - 1) / pl.Ts;
  return pl;
}

size_t permute_ws_bytes(const PermutePlan& pl) { return (size_t)(pl.blocks > 0 ? pl.blocks : 1) * pl.Gi * 4; }

// ------------------------------------------------ static device scratch ---
// Scratch of the allocation-free dispatch (moe_dispatch_noalloc): one
// file-scope device array; every GPU the library runs on holds its own copy,
// at its own address, until the process ends.  In host code `scratch` names
// a host-side stand-in, not device memory, so it is never passed to a kernel
// or a copy: the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_dispatch(const PermutePlan& pl, const int32_t* topk_idx, const int32_t* src_block,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                           const void* x, int64_t row_bytes, void* x_perm, int32_t* ws, hipStream_t s) {
  int nbits = 1;
  while ((1 << nbits) < pl.Gi) ++nbits;
  const int chunk = pl.Tc * pl.k;
  if (pl.M == 0 || pl.scanned) {
    if (pl.blocks > 0)
      seg_count_kernel<<<pl.blocks, kPermThreads, 0, s>>>(topk_idx, src_block, pl.base, pl.EL, pl.k, pl.R, pl.G,
                                                          pl.Gi, chunk, ws);
    // with no tokens this only writes zero counts and offsets
    seg_scan_kernel<<<1, kMaxSegments, 0, s>>>(pl.Gi, pl.G, pl.blocks, pl.R, ws, counts, offsets);
    if (pl.M == 0) return hipGetLastError();
  } else {
    seg_count_kernel<<<pl.blocks, kPermThreads, 0, s>>>(topk_idx, src_block, pl.base, pl.EL, pl.k, pl.R, pl.G,
                                                        pl.Gi, chunk, ws);
  }
  DispatchArgs a;
  a.topk_idx = topk_idx;
  a.src_block = src_block;
  a.ebase = pl.base;
  a.EL = pl.EL;
  a.k = pl.k;
  a.G = pl.G;
  a.Gi = pl.Gi;
  a.nbits = nbits;
  a.M = pl.M;
  a.Tc = pl.Tc;
  a.Ts = pl.Ts;
  a.chunks = pl.blocks;
  a.hist = ws;
  a.counts = counts;
  a.offsets = offsets;
  a.s2f = sorted_to_flat;
  a.f2s = flat_to_sorted;
  a.x = x_perm ? reinterpret_cast<const u32x4_t*>(x) : nullptr;
  a.xp = reinterpret_cast<u32x4_t*>(x_perm);
  a.C = (int)(row_bytes / 16);
  const dim3 grid((unsigned)pl.wgs), block(kPermThreads);
  // the narrowest register batch that holds a row's share of each thread
  const int upr = a.C <= kPermThreads ? 1 : a.C <= 2 * kPermThreads ? 2 : a.C <= 4 * kPermThreads ? 4 : 0;
  if (pl.scanned) {
    switch (upr) {
      case 1: dispatch_kernel<true, 1><<<grid, block, 0, s>>>(a); break;
      case 2: dispatch_kernel<true, 2><<<grid, block, 0, s>>>(a); break;
      case 4: dispatch_kernel<true, 4><<<grid, block, 0, s>>>(a); break;
      default: dispatch_kernel<true, 0><<<grid, block, 0, s>>>(a); break;
    }
  } else {
    switch (upr) {
      case 1: dispatch_kernel<false, 1><<<grid, block, 0, s>>>(a); break;
      case 2: dispatch_kernel<false, 2><<<grid, block, 0, s>>>(a); break;
      case 4: dispatch_kernel<false, 4><<<grid, block, 0, s>>>(a); break;
      default: dispatch_kernel<false, 0><<<grid, block, 0, s>>>(a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe

// bf16 MFMA tile of the grouped GEMM (gfx950), shared by the stand-alone
// grouped GEMM and the fused layer so both produce identical bits.
//
// What it computes ("Grouped GEMM 为什么适合 MoE": C_i = A_i B_i per expert;
// COMET paper review §3.2: Layer0 = gate/up, Layer1 = down; PTO MoE
// article: GMM1 -> SwiGLU -> GMM2):
//   layer 0: Hact[r, f] = bf16( silu(X[r]·Wg[e,f]) * (X[r]·Wu[e,f]) )
//            (silu with the hardware exp2 / reciprocal, see silu_mul_fast)
//   layer 1: Y[r, n]    = Hact[r]·Wd[e,n]            (f32)
// with every product accumulated in f32 by the matrix cores, k increasing.
//
// Design for CDNA4:
//  * The tile is 256 weight rows x TM token rows (TM = 256, or 128 for a
//    half tile), K stepped by 64.  The weight rows are the MFMA "A" operand
//    and the token rows the "B" operand, so each lane's accumulators hold 4
//    consecutive output columns of one token row: the epilogue stores 8 B
//    (bf16) / 16 B (f32) vectors.  A half tile computes every element the
//    same way as a full tile (same k order), so which height covers a row
//    never changes a bit of the result.
//  * Layer0's 256 weight rows are 128 gate rows and the 128 up rows of the
//    same columns, so a lane holds gate and up for the same (r, f) and the
//    SwiGLU runs in registers before the single bf16 store.
//  * 4 waves in a 2 x 2 arrangement, 128 x TM/2 per wave = 4 x TM/64 blocks
//    of v_mfma_f32_32x32x16_bf16 (up to 256 f32 accumulators per lane).
//  * Operands stream HBM -> VGPR (buffer loads whose range check returns 0
//    past the segment end, so ragged row tiles need no masking) -> LDS,
//    double-buffered ("Double-buffer pipeline": the next K slice loads while
//    the matrix cores work on the current one), one barrier per K step.
//  * LDS rows are 128 B; 16-byte chunk c of row r is stored at slot
//    c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1).  A ds_read_b128 of 32
//    consecutive rows then hits distinct 16-byte bank groups in every group
//    of 16 lanes (64 banks: rows r and r+1 share a 256-byte bank line) and
//    in every group of 8 lanes (32 banks).
#pragma once

#include "common.hpp"


namespace moe {

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;                           // K elements per step (128 B per row)
constexpr int kTileRows = 256;                    // weight rows and token rows per tile
constexpr int kOperandBytes = kTileRows * kBK * 2;  // 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;     // weights + tokens
constexpr int kGemmLdsBytes = 2 * kStageBytes;     // two stages: 128 KiB
constexpr int kL0Cols = 128;                       // Hact columns per layer-0 tile
constexpr int kL1Cols = 256;                       // Y columns per layer-1 tile

typedef int i32x4_t __attribute__((ext_vector_type(4)));

struct Bf16GemmArgs {
  const __bf16* a;   // token rows [R, K]; gather mode: token-major x [M, K]
  const __bf16* w0;  // layer 0: W_gate [E, F, H]; layer 1: W_down [E, H, F]
  const __bf16* w1;  // layer 0: W_up [E, F, H]
  void* c;           // layer 0: Hact [R, F] bf16 (or MXFP8 codes); layer 1: Y [R, H] f32
  // MXFP8 (one e8m0 scale byte per 32 values along the reduction index,
  // stored in groups of 32 rows: the byte of row r, block b of a tensor of
  // `cols` columns sits at (r / 32) * cols + (b / 4) * 128 + (r % 32) * 4 +
  // b % 4): layer 0 writes Hact's scales here; layer 1 reads the token rows'
  // and the weights' scales (regions of a_scale_bytes and w_scale_bytes)
  uint8_t* c_scale;
  const uint8_t* a_scale;
  const uint8_t* w_scale;
  uint32_t a_scale_bytes, w_scale_bytes;
  int K, N, E;
  // gather mode (layer 0 inside the fused layer): sorted row r reads token
  // row sorted_to_flat[r] / topk of x directly, so X_perm need not be written
  const int32_t* s2f;
  int topk;
  int64_t M;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// PARTIAL (layer 1): compute only K steps [k0, k1) and store the raw f32
// accumulators of the tile to part[t * 256 + w] (t = tile token row < trows,
// w = the tile's weight row); the caller adds the K ranges of a tile in a
// fixed order.  Otherwise k0 = 0, k1 = K / kBK (the whole reduction).
//
// OUT8 (layer 0): Hact is written as MXFP8 instead of bf16: e4m3 codes and,
// per 32 columns of a token row, one scale byte (see mx_scale / e4m3_pack4).
//
// ROWMAP: the tile's token rows are not contiguous; rowpos[t] (LDS, t < TM)
// holds the row (of a and of c) of tile row t, or -1 past the rows: a
// segment made of the rows of several source blocks for one expert, whose
// rows lie apart in the sorted order.  seg_rows and m0 then count the rows
// of that combined segment, and seg_start is unused.
template <int LAYER, bool GATHER = false, int TM = kTileRows, bool PARTIAL = false, bool OUT8 = false,
          bool ROWMAP = false>
__device__ __forceinline__ void bf16_gemm_tile(const Bf16GemmArgs& p, int g, int seg_start, int seg_rows, int m0,
                                               int nt, char* __restrict__ lds, int k0 = 0, int k1 = -1,
                                               float* __restrict__ part = nullptr,
                                               const int* __restrict__ rowpos = nullptr) {
  static_assert(!ROWMAP || (!GATHER && !PARTIAL && !OUT8), "row map: plain bf16 tiles");
  static_assert(TM == 256 || TM == 128, "token tile height");
  static_assert(!PARTIAL || (TM == 256 && LAYER == 1), "partial tiles: layer 1, full height");
  static_assert(!OUT8 || (LAYER == 0 && !PARTIAL), "MXFP8 output: layer 0");
  constexpr int NJ = TM / 64;      // token fragments per wave
  constexpr int XI = TM / 32;      // token-row loads per thread per K step
  constexpr int XQ = XI / 4;       // ... per sub-step
  // tile coordinates come from LDS; make them provably wave-uniform so the
  // buffer descriptors live in SGPRs (no per-lane descriptor loops)
  g = uniform(g);
  seg_start = uniform(seg_start);
  seg_rows = uniform(seg_rows);
  m0 = uniform(m0);
  nt = uniform(nt);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int e = g % p.E;
  const int K = p.K, N = p.N;
  const uint32_t row_bytes = (uint32_t)K * 2u;

  // ---- global -> register loads: thread owns 16-byte chunk lc of rows lr + 32 i
  const int lc = tid & 7, lr = tid >> 3;
  const int col0 = nt * (LAYER == 0 ? kL0Cols : kL1Cols);
  const int64_t ebase = (int64_t)e * N * K;
  __amdgpu_buffer_rsrc_t rw0, rw1;
  if (LAYER == 0) {
    const int ncols = min(N - col0, kL0Cols);
    rw0 = make_rsrc(p.w0 + ebase + (int64_t)col0 * K, (uint32_t)ncols * row_bytes);
    rw1 = make_rsrc(p.w1 + ebase + (int64_t)col0 * K, (uint32_t)ncols * row_bytes);
  } else {
    const int ncols = min(N - col0, kL1Cols);
    rw0 = make_rsrc(p.w0 + ebase + (int64_t)col0 * K, (uint32_t)ncols * row_bytes);
    rw1 = rw0;
  }
  const int trows = min(seg_rows - m0, TM);
  const uint32_t voff0 = (uint32_t)lr * row_bytes + (uint32_t)lc * 16u;
  const uint32_t vstep = 32u * row_bytes;
  __amdgpu_buffer_rsrc_t rx;
  uint32_t xvoff[XI];
  if (GATHER) {
    // token rows of x; rows past the segment end read zeros (offset past the range)
    rx = make_rsrc(p.a, (uint32_t)(p.M * (int64_t)row_bytes));
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int r = lr + 32 * i;
      xvoff[i] = 0x80000000u;
      if (r < trows) xvoff[i] = (uint32_t)(p.s2f[seg_start + m0 + r] / p.topk) * row_bytes + (uint32_t)lc * 16u;
    }
  } else if (ROWMAP) {
    // rows of a at their own positions (p.M rows in all); -1 reads zeros
    rx = make_rsrc(p.a, (uint32_t)(p.M * (int64_t)row_bytes));
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int r = rowpos[lr + 32 * i];
      xvoff[i] = r >= 0 ? (uint32_t)r * row_bytes + (uint32_t)lc * 16u : 0x80000000u;
    }
  } else {
    rx = make_rsrc(p.a + (int64_t)(seg_start + m0) * K, (uint32_t)trows * row_bytes);
#pragma unroll
    for (int i = 0; i < XI; ++i) xvoff[i] = voff0 + (uint32_t)i * vstep;
  }
  const uint32_t st_off = (uint32_t)lr * 128u + ((uint32_t)(lc ^ (lr & 7) ^ ((lr >> 3) & 1)) << 4);

  // Global loads in 4 parts (one per k16 sub-step of the MFMA loop); part q
  // covers the thread's weight rows lr + 32 i, i in {2q, 2q+1}, and token
  // rows lr + 32 i, i in [q XQ, (q+1) XQ).
  // With `pin`, each load is fenced from the scheduler so the loads issue in
  // source order: the prologue must issue stage 1 in the loop body's order,
  // or the wait-count pass, which merges the prologue and the loop's back
  // edge at the loop header, makes every iteration wait for the later loads.
  i32x4_t wreg[8], xreg[XI];
  auto gload_part = [&](int kt, int q, bool pin = false) {
    const uint32_t soff = (uint32_t)kt * (kBK * 2);
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) {
      if (LAYER == 0)
        wreg[i] = buf_load16(i < 4 ? rw0 : rw1, voff0 + (uint32_t)(i & 3) * vstep, soff);
      else
        wreg[i] = buf_load16(rw0, voff0 + (uint32_t)i * vstep, soff);
      if (pin) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = q * XQ; i < (q + 1) * XQ; ++i) {
      xreg[i] = buf_load16(rx, xvoff[i], soff);
      if (pin) __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto lstore_part = [&](int stage, int q) {
    char* wdst = lds + stage * kStageBytes + st_off;
    char* xdst = wdst + kOperandBytes;
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) *reinterpret_cast<i32x4_t*>(wdst + i * 4096) = wreg[i];
#pragma unroll
    for (int i = q * XQ; i < (q + 1) * XQ; ++i) *reinterpret_cast<i32x4_t*>(xdst + i * 4096) = xreg[i];
  };
  // single operations of part q (TM = 256: 2 weight and 2 token rows each),
  // for schedules that interleave stores, loads and fragment reads one by one
  auto lstore_one = [&](int stage, int q, int j) {
    char* wdst = lds + stage * kStageBytes + st_off;
    if (j < 2)
      *reinterpret_cast<i32x4_t*>(wdst + (2 * q + j) * 4096) = wreg[2 * q + j];
    else
      *reinterpret_cast<i32x4_t*>(wdst + kOperandBytes + (q * XQ + j - 2) * 4096) = xreg[q * XQ + j - 2];
  };
  auto gload_one = [&](int kt, int q, int j) {
    const uint32_t soff = (uint32_t)kt * (kBK * 2);
    if (j < 2) {
      const int i = 2 * q + j;
      if (LAYER == 0)
        wreg[i] = buf_load16(i < 4 ? rw0 : rw1, voff0 + (uint32_t)(i & 3) * vstep, soff);
      else
        wreg[i] = buf_load16(rw0, voff0 + (uint32_t)i * vstep, soff);
    } else {
      const int i = q * XQ + j - 2;
      xreg[i] = buf_load16(rx, xvoff[i], soff);
    }
  };

  // ---- fragment addressing
  const int lrow = lane & 31, lk = lane >> 5;
  uint32_t wrow_off[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int r = (LAYER == 0) ? (mi < 2 ? wn * 64 + mi * 32 : 128 + wn * 64 + (mi - 2) * 32) + lrow
                               : wn * 128 + mi * 32 + lrow;
    wrow_off[mi] = (uint32_t)r * 128u;
  }
  const uint32_t xrow_off = (uint32_t)(kOperandBytes + (wm * (TM / 2) + lrow) * 128);
  uint32_t kswz[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kswz[ks] = (uint32_t)(((2 * ks + lk) ^ (lrow & 7) ^ ((lrow >> 3) & 1)) << 4);

  // two register sets of fragments: sub-step ks uses set ks & 1 while the
  // reads for ks + 1 fill the other set
  bf16x8_t fa[2][4], fb[2][NJ];
  // fragment j of sub-step ks in the order the MFMAs use them: weight 0,
  // the token fragments, weights 1..3
  auto read_one = [&](int set, int stage, int ks, int j) {
    const char* base = lds + stage * kStageBytes;
    if (j == 0)
      fa[set][0] = *reinterpret_cast<const bf16x8_t*>(base + wrow_off[0] + kswz[ks]);
    else if (j <= NJ)
      fb[set][j - 1] = *reinterpret_cast<const bf16x8_t*>(base + xrow_off + (j - 1) * 4096 + kswz[ks]);
    else
      fa[set][j - NJ] = *reinterpret_cast<const bf16x8_t*>(base + wrow_off[j - NJ] + kswz[ks]);
  };
  auto read_frags = [&](int set, int stage, int ks) {
    const char* base = lds + stage * kStageBytes;
    // in the order the next sub-step's MFMAs (weight fragment outer) use them
    fa[set][0] = *reinterpret_cast<const bf16x8_t*>(base + wrow_off[0] + kswz[ks]);
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
      fb[set][nj] = *reinterpret_cast<const bf16x8_t*>(base + xrow_off + nj * 4096 + kswz[ks]);
#pragma unroll
    for (int mi = 1; mi < 4; ++mi)
      fa[set][mi] = *reinterpret_cast<const bf16x8_t*>(base + wrow_off[mi] + kswz[ks]);
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][nj][v] = 0.0f;

  auto mfma_rows = [&](int set, int mi0, int mi1) {
#pragma unroll
    for (int mi = mi0; mi < mi1; ++mi)
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][mi], fb[set][nj], acc[mi][nj], 0, 0, 0);
  };

  // K steps [kb, nk) of 64
  const int nk = uniform(k1 < 0 ? K / kBK : k1);
  const int kb = uniform(k0);
  // prologue: stage kb into LDS, stage kb + 1 into registers, fragments of (kb, 0)
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_part(kb, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) lstore_part(0, q);
  const int kb1 = nk > kb + 1 ? kb + 1 : kb;
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_part(kb1, q, true);
  __syncthreads();
  read_frags(0, 0, 0);

  // Main loop.  Iteration kt computes stage kt from LDS buffer kt & 1 while
  // (a) the registers holding stage kt+1 drain into the other buffer and
  // (b) the registers refill with stage kt+2 from HBM/L2, a quarter per
  // sub-step, so neither the LDS writes nor the loads sit in one burst.
  // The barrier comes before the last sub-step's second half of MFMAs: the
  // reads of the next stage's first fragments are then in flight while
  // those MFMAs run.  The last iteration's stores, loads and reads run too
  // (on a clamped, valid slice into the idle buffer) so the loop body has
  // no branches; every LDS access of the tile precedes its last barrier, so
  // the next tile's prologue may overwrite either buffer.
  //
  // One wave per SIMD cannot hide an LDS read behind another wave, so the
  // order inside each k16 sub-step is pinned with scheduling groups: the
  // MFMAs of sub-step ks alternate with the fragment reads of ks + 1, the LDS
  // stores of stage kt+1 and the loads of stage kt+2.
  constexpr int NR = 4 + NJ;        // fragment reads per sub-step
  constexpr int NW = 2 + XQ;        // LDS stores (and loads) per sub-step
  constexpr int NM = 4 * NJ;        // MFMAs per sub-step
  for (int kt = kb; kt < nk; ++kt) {
    const int cur = (kt - kb) & 1, nxt = cur ^ 1;
    const int kload = (kt + 2 < nk) ? kt + 2 : nk - 1;
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      if constexpr (TM == 256) {
        // source order = issue order: LDS operations keep their order (the
        // compiler cannot tell the two buffers apart)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          read_one((ks + 1) & 1, cur, ks + 1, 2 * j);
          lstore_one(nxt, ks, j);
          read_one((ks + 1) & 1, cur, ks + 1, 2 * j + 1);
          gload_one(kload, ks, j);
        }
      } else {
        read_frags((ks + 1) & 1, cur, ks + 1);
        lstore_part(nxt, ks);
        gload_part(kload, ks);
      }
      mfma_rows(ks & 1, 0, 4);
      if constexpr (TM == 256) {
        // one memory operation after every MFMA: fragment reads in the even
        // slots, LDS stores in slots 1, 5, 9, 13, loads in 3, 7, 11, 15 (a
        // burst of LDS stores stalls the matrix core of the issuing wave)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
      } else {
        // 8 MFMAs for 6 reads, 3 stores, 3 loads
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 3: first half of the MFMAs with the last stores and loads
    lstore_part(nxt, 3);
    gload_part(kload, 3);
    mfma_rows(1, 0, 2);
    if constexpr (TM == 256) {
      // the stores first (they must land before the barrier), then the loads
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
    } else {
#pragma unroll
      for (int i = 0; i < NM / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x220, 1, 0);  // DS write or VMEM read
      }
      if constexpr (2 * NW > NM / 2) __builtin_amdgcn_sched_group_barrier(0x220, 2 * NW - NM / 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, nxt, 0);
    mfma_rows(1, 2, 4);
#pragma unroll
    for (int i = 0; i < NM / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    if constexpr (NR > NM / 2) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM / 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue.  Lane (lrow, lk) holds, per token fragment nj and weight
  // fragment mi, the 4-column groups 8q + 4 lk (q = 0..3) of token row
  // wm*TM/2 + 32 nj + lrow.  Stored straight from there, every store would
  // touch 32 rows; the tile is staged through LDS instead, so each wave
  // stores whole 256 B (Hact) or 1 KiB (Y) row segments.  After the loop's
  // last barrier no wave reads a value from either LDS buffer again (the
  // next-stage reads of the last iteration are discarded), so both are free.
  if (PARTIAL) {
    // raw accumulators, staged as in the layer-1 epilogue: two passes of 128
    // rows, 1 KiB per staged row (256 f32 values, one per weight row of the
    // tile); 16-byte unit u of staged row t' at unit u ^ (t' & 15)
    char* stg = lds;
#pragma unroll
    for (int P = 0; P < 2; ++P) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nj = 2 * P + j;
        const int ts = wm * 64 + j * 32 + lrow;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int wb = wn * 32 + mi * 8;  // first weight row of fragment mi, in 4-row units
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = acc[mi][nj][4 * q + v];
            const int u = wb + 2 * q + lk;
            *reinterpret_cast<f32x4_t*>(stg + ts * 1024 + ((u ^ (ts & 15)) << 4)) = o;
          }
        }
      }
      __syncthreads();
      const int c = tid & 63;
#pragma unroll 4
      for (int ts = tid >> 6; ts < 128; ts += kGemmThreads / 64) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + ts * 1024 + ((c ^ (ts & 15)) << 4));
        const int trow = (ts >> 6) * (TM / 2) + 64 * P + (ts & 63);
        if (trow < trows) *reinterpret_cast<f32x4_t*>(part + (int64_t)trow * 256 + 4 * c) = v;
      }
      __syncthreads();
    }
  } else if (LAYER == 0 && OUT8) {
    // MXFP8: h (f32) is staged as 512 B per row (128 columns; 16-byte unit
    // u of row t at u ^ (t & 31)), then each thread quantises one block of
    // 32 columns of a row: the block's largest magnitude, its scale, 32
    // codes.  Four threads cover a row, so the 128 code bytes of a row are
    // stored contiguously.
    char* stg = lds;
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      const int t = wm * (TM / 2) + nj * 32 + lrow;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t h;
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = silu_mul_fast(acc[mi][nj][4 * q + v], acc[mi + 2][nj][4 * q + v]);
          const int u = wn * 16 + mi * 8 + 2 * q + lk;
          *reinterpret_cast<f32x4_t*>(stg + t * 512 + ((u ^ (t & 31)) << 4)) = h;
        }
      }
    }
    __syncthreads();
    uint8_t* hact = reinterpret_cast<uint8_t*>(p.c);
    const int b = tid & 3;
    const int f = col0 + 32 * b;
    for (int t = tid >> 2; t < TM; t += kGemmThreads / 4) {
      f32x4_t v[8];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = *reinterpret_cast<const f32x4_t*>(stg + t * 512 + (((8 * b + j) ^ (t & 31)) << 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
      }
      const int X = mx_scale(amax);
      i32x4_t out[2];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        out[j / 4][j % 4] = (int)e4m3_pack4(ldexpf(v[j][0], -X), ldexpf(v[j][1], -X), ldexpf(v[j][2], -X),
                                            ldexpf(v[j][3], -X));
      const int trow = m0 + t;
      if (trow < seg_rows && f < N) {
        uint8_t* dst = hact + (int64_t)(seg_start + trow) * N + f;
        *reinterpret_cast<i32x4_t*>(dst) = out[0];
        *reinterpret_cast<i32x4_t*>(dst + 16) = out[1];
        const int64_t r = seg_start + trow;
        p.c_scale[(r >> 5) * N + col0 + (r & 31) * 4 + b] = (uint8_t)(X + 127);
      }
    }
    __syncthreads();
  } else if (LAYER == 0) {
    // 256 B per staged row (128 bf16 columns); 8-byte unit u of row t at
    // unit u ^ (t & 31): conflict-free for 32 rows writing the same unit.
    char* stg = lds;
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      const int t = wm * (TM / 2) + nj * 32 + lrow;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4_t h;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gt = acc[mi][nj][4 * q + v], up = acc[mi + 2][nj][4 * q + v];
            h[v] = (__bf16)silu_mul_fast(gt, up);
          }
          const int u = wn * 16 + mi * 8 + 2 * q + lk;
          *reinterpret_cast<bf16x4_t*>(stg + t * 256 + ((u ^ (t & 31)) << 3)) = h;
        }
      }
    }
    __syncthreads();
    // 16 threads per row, 16 B (8 columns) each: chunk c of row t sits at
    // chunk c ^ ((t & 31) >> 1), its two halves swapped when t is odd.
    __bf16* hact = reinterpret_cast<__bf16*>(p.c);
    const int c = tid & 15;
    const int f = col0 + 8 * c;
#pragma unroll 4
    for (int t = tid >> 4; t < TM; t += kGemmThreads / 16) {
      i32x4_t v = *reinterpret_cast<const i32x4_t*>(stg + t * 256 + ((c ^ ((t & 31) >> 1)) << 4));
      if (t & 1) v = i32x4_t{v[2], v[3], v[0], v[1]};
      const int trow = m0 + t;
      if (trow < seg_rows && f < N)
        *reinterpret_cast<i32x4_t*>(hact + (int64_t)(ROWMAP ? rowpos[t] : seg_start + trow) * N + f) = v;
    }
    __syncthreads();
  } else {
    // Two passes of 128 rows (one for a half tile), 1 KiB per staged row (256
    // f32 columns) over both buffers; 16-byte unit u of staged row t' at unit
    // u ^ (t' & 15).  Pass P stages token fragments nj = 2P, 2P + 1: staged
    // row t' = wm*64 + (nj & 1)*32 + lrow is tile row wm*TM/2 + 64 P + t' % 64.
    float* y = reinterpret_cast<float*>(p.c);
    char* stg = lds;
    constexpr int passes = NJ / 2;
#pragma unroll
    for (int P = 0; P < passes; ++P) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nj = 2 * P + j;
        const int ts = wm * 64 + j * 32 + lrow;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = acc[mi][nj][4 * q + v];
            const int u = wn * 32 + mi * 8 + 2 * q + lk;
            *reinterpret_cast<f32x4_t*>(stg + ts * 1024 + ((u ^ (ts & 15)) << 4)) = o;
          }
        }
      }
      __syncthreads();
      // 64 threads per staged row, 16 B (4 columns) each
      const int c = tid & 63;
      const int n = col0 + 4 * c;
#pragma unroll 4
      for (int ts = tid >> 6; ts < 128; ts += kGemmThreads / 64) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + ts * 1024 + ((c ^ (ts & 15)) << 4));
        const int t = (ts >> 6) * (TM / 2) + 64 * P + (ts & 63);
        const int trow = m0 + t;
        if (trow < seg_rows && n < N)
          *reinterpret_cast<f32x4_t*>(y + (int64_t)(ROWMAP ? rowpos[t] : seg_start + trow) * N + n) = v;
      }
      __syncthreads();
    }
  }
}

// One row tile of a segment.  A segment of at most 128 rows (its only row
// tile) runs as the 128-row variant: half the matrix-core work, the same k
// order per element, so the same bits.  Longer segments' last tiles stay
// full height: then every tile of a segment takes the same time, the tiles
// running at once on an XCD stay in step and share the segment's weight
// panels in its L2 (measured: halving those last tiles cost more in
// re-read weights than it saved).
template <int LAYER, bool GATHER = false, bool OUT8 = false, bool ROWMAP = false>
__device__ __forceinline__ void bf16_gemm_row_tile(const Bf16GemmArgs& p, int g, int seg_start, int seg_rows, int m0,
                                                   int nt, char* __restrict__ lds,
                                                   const int* __restrict__ rowpos = nullptr) {
  if (seg_rows <= kTileRows / 2)
    bf16_gemm_tile<LAYER, GATHER, kTileRows / 2, false, OUT8, ROWMAP>(p, g, seg_start, seg_rows, m0, nt, lds, 0, -1,
                                                                      nullptr, rowpos);
  else
    bf16_gemm_tile<LAYER, GATHER, kTileRows, false, OUT8, ROWMAP>(p, g, seg_start, seg_rows, m0, nt, lds, 0, -1,
                                                                  nullptr, rowpos);
}

}  // namespace moe

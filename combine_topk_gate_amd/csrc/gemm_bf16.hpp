// bf16 MFMA tile of the grouped GEMM (gfx950), shared by the stand-alone
// grouped GEMM and the fused layer so both produce identical bits.
//
// What it computes ("Grouped GEMM 为什么适合 MoE": C_i = A_i B_i per expert;
// COMET paper review §3.2: Layer0 = gate/up, Layer1 = down; PTO MoE
// article: GMM1 -> SwiGLU -> GMM2):
//   layer 0: Hact[r, f] = bf16( silu(X[r]·Wg[e,f]) * (X[r]·Wu[e,f]) )
//   layer 1: Y[r, n]    = Hact[r]·Wd[e,n]            (f32)
// with every product accumulated in f32 by the matrix cores, k increasing.
//
// Design for CDNA4:
//  * The tile is 256 weight rows x 256 token rows, K stepped by 64.  The
//    weight rows are the MFMA "A" operand and the token rows the "B"
//    operand, so each lane's accumulators hold 4 consecutive output columns
//    of one token row: the epilogue stores 8 B (bf16) / 16 B (f32) vectors.
//  * Layer0's 256 weight rows are 128 gate rows and the 128 up rows of the
//    same columns, so a lane holds gate and up for the same (r, f) and the
//    SwiGLU runs in registers before the single bf16 store.
//  * 4 waves in a 2 x 2 arrangement, 128 x 128 per wave = 4 x 4 blocks of
//    v_mfma_f32_32x32x16_bf16 (256 f32 accumulators per lane).
//  * Operands stream HBM -> VGPR (buffer loads whose range check returns 0
//    past the segment end, so ragged row tiles need no masking) -> LDS,
//    double-buffered ("Double-buffer pipeline": the next K slice loads while
//    the matrix cores work on the current one), one barrier per K step.
//  * LDS rows are 128 B; 16-byte chunk c of row r is stored at slot
//    c ^ (r & 7), so the 8 lanes of each ds_read_b128 phase hit 8 different
//    bank groups.
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
  const __bf16* a;   // token rows [R, K]
  const __bf16* w0;  // layer 0: W_gate [E, F, H]; layer 1: W_down [E, H, F]
  const __bf16* w1;  // layer 0: W_up [E, F, H]
  void* c;           // layer 0: Hact [R, F] bf16; layer 1: Y [R, H] f32
  int K, N, E;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

template <int LAYER>
__device__ __forceinline__ void bf16_gemm_tile(const Bf16GemmArgs& p, int g, int seg_start, int seg_rows, int m0,
                                               int nt, char* __restrict__ lds) {
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
  const int trows = min(seg_rows - m0, kTileRows);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.a + (int64_t)(seg_start + m0) * K, (uint32_t)trows * row_bytes);

  const uint32_t voff0 = (uint32_t)lr * row_bytes + (uint32_t)lc * 16u;
  const uint32_t vstep = 32u * row_bytes;
  const uint32_t st_off = (uint32_t)lr * 128u + ((uint32_t)(lc ^ (lr & 7)) << 4);

  i32x4_t wreg[8], xreg[8];
  auto gload = [&](int kt) {
    const uint32_t soff = (uint32_t)kt * (kBK * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (LAYER == 0)
        wreg[i] = buf_load16(i < 4 ? rw0 : rw1, voff0 + (uint32_t)(i & 3) * vstep, soff);
      else
        wreg[i] = buf_load16(rw0, voff0 + (uint32_t)i * vstep, soff);
      xreg[i] = buf_load16(rx, voff0 + (uint32_t)i * vstep, soff);
    }
  };
  auto lstore = [&](int stage) {
    char* wdst = lds + stage * kStageBytes + st_off;
    char* xdst = wdst + kOperandBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<i32x4_t*>(wdst + i * 4096) = wreg[i];
      *reinterpret_cast<i32x4_t*>(xdst + i * 4096) = xreg[i];
    }
  };

  // ---- fragment addressing
  const int lrow = lane & 31, lk = lane >> 5;
  int wrow[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (LAYER == 0)
      wrow[mi] = (mi < 2 ? wn * 64 + mi * 32 : 128 + wn * 64 + (mi - 2) * 32) + lrow;
    else
      wrow[mi] = wn * 128 + mi * 32 + lrow;
  }
  const int xrow0 = wm * 128 + lrow;
  uint32_t kswz[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kswz[ks] = (uint32_t)(((2 * ks + lk) ^ (lrow & 7)) << 4);

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][nj][v] = 0.0f;

  const int nk = K / kBK;
  gload(0);
  lstore(0);
  if (nk > 1) gload(1);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const char* wsrc = lds + (kt & 1) * kStageBytes;
    const char* xsrc = wsrc + kOperandBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(wsrc + wrow[mi] * 128 + kswz[ks]);
#pragma unroll
      for (int nj = 0; nj < 4; ++nj)
        bfr[nj] = *reinterpret_cast<const bf16x8_t*>(xsrc + (xrow0 + nj * 32) * 128 + kswz[ks]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      lstore((kt + 1) & 1);
      if (kt + 2 < nk) gload(kt + 2);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds column block 8q + 4 lk + (0..3) of token row lrow
  if (LAYER == 0) {
    __bf16* hact = reinterpret_cast<__bf16*>(p.c);
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
      const int trow = m0 + wm * 128 + nj * 32 + lrow;
      if (trow >= seg_rows) continue;
      __bf16* dst = hact + (int64_t)(seg_start + trow) * N;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = col0 + wn * 64 + mi * 32 + 8 * q + 4 * lk;
          if (f >= N) continue;
          bf16x4_t h;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gt = acc[mi][nj][4 * q + v], up = acc[mi + 2][nj][4 * q + v];
            h[v] = (__bf16)(silu_f32(gt) * up);
          }
          *reinterpret_cast<bf16x4_t*>(dst + f) = h;
        }
      }
    }
  } else {
    float* y = reinterpret_cast<float*>(p.c);
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
      const int trow = m0 + wm * 128 + nj * 32 + lrow;
      if (trow >= seg_rows) continue;
      float* dst = y + (int64_t)(seg_start + trow) * N;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = col0 + wn * 128 + mi * 32 + 8 * q + 4 * lk;
          if (n >= N) continue;
          f32x4_t o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = acc[mi][nj][4 * q + v];
          *reinterpret_cast<f32x4_t*>(dst + n) = o;
        }
      }
    }
  }
}

}  // namespace moe

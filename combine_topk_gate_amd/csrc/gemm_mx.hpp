// Layer1 grouped-GEMM tile on MXFP8 operands (matrix cores, gfx950).
//
// PTO MoE article, two-stage SwiGLU: the activation is quantised as SwiGLU
// produces it and the down product consumes the quantised values.  Both
// operands are in the OCP microscaling format MXFP8: e4m3 codes and one
// power-of-two scale byte per 32 values along the reduction index F (Hact
// [R, F], W_down [E, H, F] as [E*H, F]).  The scale bytes are stored in
// groups of 32 rows: per group and 128-column quad (one stage), the 4 bytes
// of each row in turn, so the scales of 32 fragment rows for a stage are
// one 128-byte line.
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies the codes and applies both
// operands' block scales itself, so nothing is dequantised in registers.
//
// The tile is the bf16 tile's (256 weight rows x TM token rows, 4 waves of
// 128 x TM/2, LDS double buffer, the same 16-byte-chunk swizzle): a stage of
// 128 fp8 values is 128 bytes per row, exactly a bf16 stage of 64, so the
// loads and the LDS layout are unchanged and each stage carries twice the
// products.  Per stage a wave runs two k64 sub-steps of 4 x NJ MFMAs.
//
// Operand layout of the 32x32x64 fp8 MFMA (measured on the device): lane
// l = 32 h + i holds row i; its bytes 0..15 are k = 16 h .. 16 h + 15 and
// bytes 16..31 are k = 32 + 16 h .. 32 + 16 h + 15 of the sub-step, so every
// lane's first 16 bytes lie in scale block 0 and the rest in block 1; the
// scale of block b of row i is taken from lane 32 b + i.  The result has the
// bf16 MFMA's layout.
#pragma once

#include "gemm_bf16.hpp"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

template <int TM = kTileRows>
__device__ __forceinline__ void mx_gemm_tile(const Bf16GemmArgs& p, int g, int seg_start, int seg_rows, int m0,
                                             int nt, char* __restrict__ lds) {
  static_assert(TM == 256 || TM == 128, "token tile height");
  constexpr int NJ = TM / 64;  // token fragments per wave
  constexpr int XI = TM / 32;  // token-row loads per thread per stage
  g = uniform(g);
  seg_start = uniform(seg_start);
  seg_rows = uniform(seg_rows);
  m0 = uniform(m0);
  nt = uniform(nt);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int e = g % p.E;
  const int K = p.K, N = p.N;  // K = F (bytes per row), N = H
  const uint32_t row_bytes = (uint32_t)K;

  const int lc = tid & 7, lr = tid >> 3;
  const int col0 = nt * kL1Cols;
  const int ncols = min(N - col0, kL1Cols);
  const int trows = min(seg_rows - m0, TM);
  const uint8_t* wcodes = reinterpret_cast<const uint8_t*>(p.w0);
  const uint8_t* xcodes = reinterpret_cast<const uint8_t*>(p.a);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wcodes + ((int64_t)e * N + col0) * K, (uint32_t)ncols * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xcodes + (int64_t)(seg_start + m0) * K, (uint32_t)trows * row_bytes);
  // whole scale regions; a fragment row past the tile's rows takes an
  // offset past the region and reads scale 0 (its codes read 0 as well)
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.w_scale, p.w_scale_bytes);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.a_scale, p.a_scale_bytes);
  const uint32_t voff0 = (uint32_t)lr * row_bytes + (uint32_t)lc * 16u;
  const uint32_t vstep = 32u * row_bytes;
  const uint32_t st_off = (uint32_t)lr * 128u + ((uint32_t)(lc ^ (lr & 7) ^ ((lr >> 3) & 1)) << 4);

  i32x4_t wreg[8], xreg[XI];
  auto gload = [&](int kt) {
    const uint32_t soff = (uint32_t)kt * 128u;
#pragma unroll
    for (int i = 0; i < 8; ++i) wreg[i] = buf_load16(rw, voff0 + (uint32_t)i * vstep, soff);
#pragma unroll
    for (int i = 0; i < XI; ++i) xreg[i] = buf_load16(rx, voff0 + (uint32_t)i * vstep, soff);
  };
  auto lstore = [&](int stage) {
    char* wdst = lds + stage * kStageBytes + st_off;
    char* xdst = wdst + kOperandBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<i32x4_t*>(wdst + i * 4096) = wreg[i];
#pragma unroll
    for (int i = 0; i < XI; ++i) *reinterpret_cast<i32x4_t*>(xdst + i * 4096) = xreg[i];
  };

  // fragment rows and the swizzled offsets of the two 16-byte chunks a lane
  // reads per k64 sub-step: chunks 4 kk + lk and 4 kk + 2 + lk of the row
  const int lrow = lane & 31, lk = lane >> 5;
  uint32_t wrow_off[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) wrow_off[mi] = (uint32_t)(wn * 128 + mi * 32 + lrow) * 128u;
  const uint32_t xrow_off = (uint32_t)(kOperandBytes + (wm * (TM / 2) + lrow) * 128);
  uint32_t kswz[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      kswz[kk][c] = (uint32_t)(((4 * kk + 2 * c + lk) ^ (lrow & 7) ^ ((lrow >> 3) & 1)) << 4);

  i32x8_t fa[2][4], fb[2][NJ];
  auto read_frag = [&](const char* at, int kk) {
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(at + kswz[kk][0]);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(at + kswz[kk][1]);
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_frags = [&](int set, int stage, int kk) {
    const char* base = lds + stage * kStageBytes;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) fa[set][mi] = read_frag(base + wrow_off[mi], kk);
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) fb[set][nj] = read_frag(base + xrow_off + nj * 4096, kk);
  };

  // scale dwords (blocks 4 kt .. 4 kt + 3 of the lane's rows), shifted so
  // byte 2 kk is block 4 kt + 2 kk + lk.  Row r's dword of stage kt is at
  // (r / 32) * K + kt * 128 + (r % 32) * 4; the fragment rows of one lane
  // group are 32 consecutive rows, so a load covers one or two lines.
  uint32_t sw[4], sx[NJ], sw_n[4], sx_n[NJ];
  uint32_t sw_off[4], sx_off[NJ];
  constexpr uint32_t kNoRow = 0xC0000000u;  // past any scale region
  auto soffset = [&](int64_t r) { return (uint32_t)((r >> 5) * K + (r & 31) * 4); };
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int lr_ = wn * 128 + mi * 32 + lrow;
    sw_off[mi] = lr_ < ncols ? soffset((int64_t)e * N + col0 + lr_) : kNoRow;
  }
#pragma unroll
  for (int nj = 0; nj < NJ; ++nj) {
    const int lr_ = wm * (TM / 2) + nj * 32 + lrow;
    sx_off[nj] = lr_ < trows ? soffset((int64_t)seg_start + m0 + lr_) : kNoRow;
  }
  auto sload = [&](uint32_t* dw, uint32_t* dx, int kt) {
    const uint32_t soff = (uint32_t)kt * 128u;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) dw[mi] = buf_load4(rws, sw_off[mi], soff) >> (8 * lk);
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) dx[nj] = buf_load4(rxs, sx_off[nj], soff) >> (8 * lk);
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][nj][v] = 0.0f;

  auto mfmas = [&](int set, int kk) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int sa = (int)((sw[mi] >> (16 * kk)) & 0xFFu);
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
        const int sb = (int)((sx[nj] >> (16 * kk)) & 0xFFu);
        acc[mi][nj] =
            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[set][mi], fb[set][nj], acc[mi][nj], 0, 0, 0, sa, 0, sb);
      }
    }
  };

  const int nk = uniform(K / 128);
  // prologue: stage 0 into LDS, then the scales of stage 0 and stage 1 into
  // registers, each load fenced so they issue in the loop body's order
  // (scales, weights, tokens): the wait-count pass merges the prologue with
  // the loop's back edge at the loop header, and any other order makes every
  // iteration wait for loads it does not need yet
  gload(0);
  lstore(0);
  {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      sw[mi] = buf_load4(rws, sw_off[mi], 0) >> (8 * lk);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      sx[nj] = buf_load4(rxs, sx_off[nj], 0) >> (8 * lk);
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint32_t soff = (uint32_t)(nk > 1 ? 1 : 0) * 128u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wreg[i] = buf_load16(rw, voff0 + (uint32_t)i * vstep, soff);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      xreg[i] = buf_load16(rx, voff0 + (uint32_t)i * vstep, soff);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  read_frags(0, 0, 0);

  if constexpr (TM == kTileRows) {
    // Iteration kt, as in the bf16 tile: sub-step 0 (16 MFMAs on fragment
    // set 0) with, after each MFMA, one read of sub-step 1's fragments (set
    // 1), one of the first 8 LDS stores of stage kt+1 into the other buffer
    // and one load (the 8 scale dwords of kt+1 first, so waiting for them
    // never waits for the data loads issued after; then the weights of
    // kt+2).  Sub-step 1: the last 8 stores beside the first 8 MFMAs, the
    // barrier, then stage kt+1's first fragments (into set 0, free by now)
    // and the token loads beside the last 8 MFMAs, so the matrix cores keep
    // working across the barrier.  The order is pinned with scheduling
    // groups: one wave per SIMD cannot hide a burst of memory operations
    // behind another wave.
    constexpr int NR = 2 * (4 + NJ);  // 16-byte fragment reads per sub-step
    auto read_one = [&](int set, int stage, int kk, int j) {
      // fragments in the order the MFMAs use them: weight 0, the token
      // fragments, weights 1..3; each as two 16-byte halves
      const int f = j >> 1, c = j & 1;
      const int mi = (f == 0) ? 0 : (f <= NJ ? -1 : f - NJ);
      const char* base = lds + stage * kStageBytes;
      const char* at = (mi >= 0 ? base + wrow_off[mi] : base + xrow_off + (f - 1) * 4096) + kswz[kk][c];
      const i32x4_t v = *reinterpret_cast<const i32x4_t*>(at);
      if (mi >= 0) {
        if (c == 0) fa[set][mi].lo = v; else fa[set][mi].hi = v;
      } else {
        if (c == 0) fb[set][f - 1].lo = v; else fb[set][f - 1].hi = v;
      }
    };
    auto store_one = [&](int stage, int i) {
      char* wdst = lds + stage * kStageBytes + st_off;
      if (i < 8)
        *reinterpret_cast<i32x4_t*>(wdst + i * 4096) = wreg[i];
      else
        *reinterpret_cast<i32x4_t*>(wdst + kOperandBytes + (i - 8) * 4096) = xreg[i - 8];
    };
    auto mfma_half = [&](int set, int kk, int h) {  // weight fragments 2h, 2h + 1
#pragma unroll
      for (int mi = 2 * h; mi < 2 * h + 2; ++mi) {
        const int sa = (int)((sw[mi] >> (16 * kk)) & 0xFFu);
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
          const int sb = (int)((sx[nj] >> (16 * kk)) & 0xFFu);
          acc[mi][nj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[set][mi], fb[set][nj], acc[mi][nj], 0, 0, 0,
                                                                       sa, 0, sb);
        }
      }
    };
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1, nxt = cur ^ 1;
      const int kload = (kt + 2 < nk) ? kt + 2 : nk - 1;
      const uint32_t soff = (uint32_t)kload * 128u;
      const uint32_t ssoff = (uint32_t)((kt + 1 < nk) ? kt + 1 : nk - 1) * 128u;
      // sub-step 0: after each MFMA one read (set 1), one store (the first
      // 8 of stage kt+1) or none, and one load (scales of kt+1, then the
      // weights of kt+2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        read_one(1, cur, 1, i);
        if (i < 8) store_one(nxt, i);
        if (i < 4)
          sw_n[i] = buf_load4(rws, sw_off[i], ssoff) >> (8 * lk);
        else if (i < 8)
          sx_n[i - 4] = buf_load4(rxs, sx_off[i - 4], ssoff) >> (8 * lk);
        else
          wreg[i - 8] = buf_load16(rw, voff0 + (uint32_t)(i - 8) * vstep, soff);
      }
      mfmas(0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        if (i < 8) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
      // sub-step 1, first half (weights 0, 1): the last 8 stores
#pragma unroll
      for (int i = 8; i < 16; ++i) store_one(nxt, i);
      mfma_half(1, 1, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      // sub-step 1, second half (weights 2, 3): stage kt+1's first fragments
      // into the free set 0, and the token loads of kt+2
#pragma unroll
      for (int i = 0; i < NR; ++i) read_one(0, nxt, 0, i);
#pragma unroll
      for (int i = 0; i < XI; ++i) xreg[i] = buf_load16(rx, voff0 + (uint32_t)i * vstep, soff);
      mfma_half(1, 1, 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) sw[mi] = sw_n[mi];
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) sx[nj] = sx_n[nj];
    }
  } else {
    // half-height tiles: the same steps, scheduled by the compiler
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1, nxt = cur ^ 1;
      const int kload = (kt + 2 < nk) ? kt + 2 : nk - 1;
      read_frags(1, cur, 1);
      lstore(nxt);
      sload(sw_n, sx_n, (kt + 1 < nk) ? kt + 1 : nk - 1);
      gload(kload);
      mfmas(0, 0);
      __syncthreads();
      read_frags(0, nxt, 0);
      mfmas(1, 1);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) sw[mi] = sw_n[mi];
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) sx[nj] = sx_n[nj];
    }
  }
  // the last iteration's reads of the idle buffer finish before the
  // epilogue reuses the LDS
  __syncthreads();

  // ---- epilogue: Y rows, staged through LDS as in the bf16 Layer1 tile
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
    const int c = tid & 63;
    const int n = col0 + 4 * c;
#pragma unroll 4
    for (int ts = tid >> 6; ts < 128; ts += kGemmThreads / 64) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + ts * 1024 + ((c ^ (ts & 15)) << 4));
      const int trow = m0 + (ts >> 6) * (TM / 2) + 64 * P + (ts & 63);
      if (trow < seg_rows && n < N) *reinterpret_cast<f32x4_t*>(y + (int64_t)(seg_start + trow) * N + n) = v;
    }
    __syncthreads();
  }
}

}  // namespace moe

// Internal helpers shared by the library's HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Device-side status words kept at the start of the fused layer's workspace.
constexpr int kStatusOk = 0;
constexpr int kStatusTimeout = 5;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

// f32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// silu(g) * u for the bf16 layers' epilogue, with the hardware base-2
// exponential and reciprocal (about 1 ulp each): silu(g) = g / (1 + e^-g)
// = g * rcp(1 + 2^(-g log2 e)).  Its error (~1e-7 relative) is far below
// the bf16 rounding of the activation that follows; for g -> -inf the
// exponential saturates to +inf and the reciprocal to 0, the exact limit.
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return (g * u) * __builtin_amdgcn_rcpf(1.0f + e);
}

// MXFP8 (the OCP microscaling format with e4m3 elements): a block of 32
// values shares the scale 2^X, X = floor(log2 of the block's largest
// magnitude) - 8 (8 is the exponent of e4m3's largest value, 448), within
// [-127, 127]; -127 for an all-zero block.  The scale byte is X + 127.
__device__ __forceinline__ int mx_scale(float amax) {
  const int ef = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFF);
  if (ef == 0) return -127;  // zero, or below the smallest normal f32
  const int X = ef - 127 - 8;
  return X < -127 ? -127 : X;
}

// Scale bytes of an MXFP8 tensor of rows x cols (cols a multiple of 128):
// one per 32 values, rows padded to a multiple of 32 (groups of 32 rows;
// per group and 128-column quad, the 4 bytes of each row in turn).
__host__ __device__ __forceinline__ int64_t mx_scale_bytes(int64_t rows, int64_t cols) {
  return (rows + 31) / 32 * 32 * (cols / 32);
}

// e4m3 codes of four values already divided by the block scale (|v| <
// 512), packed little-endian: round to nearest, ties to even, magnitudes
// past 448 give 448 (0x7E), sign kept.  The values are first clamped to
// [-448, 448], so the hardware conversion (OCP e4m3 on gfx950, correctly
// rounded in the default round-to-nearest-even mode) never overflows;
// inside that range its rounding is the format's.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  auto sat = [](float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

// Top-k weighted reduction of one 4-wide column group, shared by the
// stand-alone combine and the fused layer so both give identical bits.
// A slot whose row is -1 (a pair of an expert not held here), or any row
// outside [0, R), is left out.
__device__ __forceinline__ float4 combine_group(const float* __restrict__ y, const float* __restrict__ w,
                                                const int32_t* __restrict__ rows, int k, int64_t H, int64_t n,
                                                int64_t R) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    if ((uint64_t)(int64_t)rows[j] >= (uint64_t)R) continue;
    const float wj = w[j];
    const float4 v = *reinterpret_cast<const float4*>(y + (int64_t)rows[j] * H + n);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  return acc;
}

// Output epilogue of the combine: out = cast(acc + residual), one f32 add
// (none without a residual), then f32 or bf16 (round to nearest even).
struct OutEpilogue {
  const void* residual;  // [M,H] bf16 or f32, or null
  void* out;             // [M,H] f32 or bf16
  int res_bf16;
  int out_bf16;
};

// Stores the 4 values of out starting at element i (= t * H + n, i % 4 == 0).
__device__ __forceinline__ void store_out(const OutEpilogue& ep, int64_t i, float4 acc) {
  if (ep.residual) {
    float4 r;
    if (ep.res_bf16) {
      const bf16x4_t b = *reinterpret_cast<const bf16x4_t*>(reinterpret_cast<const __bf16*>(ep.residual) + i);
      r = make_float4((float)b[0], (float)b[1], (float)b[2], (float)b[3]);
    } else {
      r = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(ep.residual) + i);
    }
    acc.x += r.x;
    acc.y += r.y;
    acc.z += r.z;
    acc.w += r.w;
  }
  if (ep.out_bf16) {
    bf16x4_t o;
    o[0] = (__bf16)acc.x;
    o[1] = (__bf16)acc.y;
    o[2] = (__bf16)acc.z;
    o[3] = (__bf16)acc.w;
    *reinterpret_cast<bf16x4_t*>(reinterpret_cast<__bf16*>(ep.out) + i) = o;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.out) + i) = acc;
  }
}

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace moe

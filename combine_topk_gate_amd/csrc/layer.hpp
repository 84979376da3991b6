// Fused MoE layer (internal interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef const int32_t* src_ptr_t;

struct FusedArgs {
  int64_t M;
  int H, F, E, k, G;
  const void* x;
  const void* x_perm;  // non-null: Layer0 reads X_perm (written by the dispatch); null: it gathers from x
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* s2f;
  const int32_t* f2s;
  void* hact;
  float* y;
  OutEpilogue out;  // out, with the optional residual and its output type
  int32_t* status;
  int32_t* flags;
  int mt_max;  // M-tile bound the flag arrays are sized for
  int grid;
  int n_mover;
  int spin_limit;
  uint32_t shuffle;  // nonzero: items in a seeded permutation inside each section (debug check)
};

size_t fused_ws_bytes(int64_t M, int H, int F, int E, int k, int S);
int fused_mt_max(int64_t M, int H, int k, int G);
// Words of the ready counters and queue counters at FusedArgs::flags; they
// must be zero when the fused kernel starts (the layer call's route kernel
// clears them).
int fused_flag_words(int64_t M, int H, int k, int G);
// EL: experts held (E when all are).  kTableUnusable: MOE_TUNING_TABLE names
// a file that cannot be read or parsed.
constexpr int kTableUnusable = -2;
int fused_default_movers(int64_t M, int H, int F, int E, int k, int S, int EL, int dtype, int cus);
moe_status_t fused_check(const FusedArgs& a, int cus);
hipError_t launch_fused_layer(const FusedArgs& a, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

}  // namespace moe

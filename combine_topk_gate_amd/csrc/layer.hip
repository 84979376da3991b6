// Fused MoE layer: placeholder until the fused kernel lands; the layer runs
// the kernel chain (route, permute, dispatch, grouped GEMM x2, combine).
#include "common.hpp"
#include "layer.hpp"

namespace moe {

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  fill_i32_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

size_t fused_ws_bytes(int64_t, int, int, int, int, int) { return 0; }

int fused_default_movers(int64_t, int, int, int, int, int, int, int) { return 0; }

moe_status_t fused_check(const FusedArgs&, int) { return MOE_ERR_UNSUPPORTED; }

hipError_t launch_fused_layer(const FusedArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe

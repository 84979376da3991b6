// C ABI of the library: host-side argument checks, workspace carving and
// kernel launches.  Every entry point only enqueues work on the caller's
// stream; none synchronises (except moe_debug_device_status, a test hook).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "common.hpp"
#include "launch.hpp"
#include "layer.hpp"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// bytes per element of x and X_perm (and of Hact unless it is MXFP8)
size_t elem_bytes(const moe_problem_t* p) { return p->dtype == MOE_DTYPE_F32 ? 4 : 2; }
bool is_mx(const moe_problem_t* p) { return p->dtype == MOE_DTYPE_BF16_MXFP8; }
// bytes of the Hact buffer: R x F elements, or an MXFP8 buffer (codes + scales)
size_t hact_bytes(const moe_problem_t* p, int64_t R) {
  return is_mx(p) ? (size_t)R * p->ffn + (size_t)mx_scale_bytes(R, p->ffn) : (size_t)R * p->ffn * elem_bytes(p);
}

// Whether the bf16 grouped GEMM combines each expert's segments of all the
// source blocks into one: with source blocks whose (block, expert)
// segments hold fewer rows than a tile on average (R EL / E kept pairs over
// S EL segments, i.e. R / (E S) < 256), such as the expert-parallel share
// that holds a few of many experts.
bool combine_blocks(const moe_problem_t* p) {
  return p->dtype == MOE_DTYPE_BF16 && p->num_src_blocks > 1 &&
         p->num_tokens * p->topk < 256ll * p->num_experts * p->num_src_blocks;
}

// Experts held by the call (weights it is given): EL, or all E.
int held(const moe_problem_t* p) { return p->local_experts > 0 ? p->local_experts : p->num_experts; }
int held_base(const moe_problem_t* p) { return p->local_experts > 0 ? p->expert_base : 0; }
// Segments: S * EL.
int segments(const moe_problem_t* p) { return p->num_src_blocks * held(p); }

moe_status_t check_problem(const moe_problem_t* p) {
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t M = p->num_tokens;
  if (M < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->hidden < 64 || p->hidden > 65536 || p->hidden % 64) return MOE_ERR_INVALID_ARGUMENT;
  if (p->ffn < 64 || p->ffn > 65536 || p->ffn % 64) return MOE_ERR_INVALID_ARGUMENT;
  if (p->num_experts < 1 || p->num_experts > 512) return MOE_ERR_INVALID_ARGUMENT;
  if (p->topk < 1 || p->topk > 16 || p->topk > p->num_experts) return MOE_ERR_INVALID_ARGUMENT;
  if (p->local_experts < 0 || p->expert_base < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->local_experts == 0 && p->expert_base != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->expert_base + p->local_experts > p->num_experts) return MOE_ERR_INVALID_ARGUMENT;
  // dropped pairs take one more segment in the bookkeeping
  const int64_t ranked = (int64_t)p->num_src_blocks * held(p) + (held(p) < p->num_experts ? 1 : 0);
  if (p->num_src_blocks < 1 || ranked > 1024) return MOE_ERR_INVALID_ARGUMENT;
  if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16 && p->dtype != MOE_DTYPE_BF16_MXFP8)
    return MOE_ERR_INVALID_ARGUMENT;
  if (p->dtype == MOE_DTYPE_BF16_MXFP8 && p->ffn % 128) return MOE_ERR_UNSUPPORTED;
  if (M >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;  // bounded before M * topk is formed
  const int64_t R = M * p->topk;
  if (R >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  const int64_t wide = p->hidden > p->ffn ? p->hidden : p->ffn;
  if (R * wide >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  // weights are addressed per expert with 64-bit offsets; the MXFP8 weight
  // scales are one buffer range of EL*H*F/32 bytes, below 2^32
  if ((int64_t)held(p) * p->hidden * p->ffn >= (1ll << 37)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

PermutePlan plan_of(const moe_problem_t* p) {
  return permute_plan(p->num_tokens, p->topk, p->num_src_blocks, p->num_experts, held_base(p), p->local_experts);
}

// Epilogue of the combine from the caller's description (null: plain f32).
moe_status_t epilogue_of(const moe_problem_t* p, const moe_epilogue_t* epi, void* out, OutEpilogue* ep) {
  ep->out = out;
  ep->residual = nullptr;
  ep->res_bf16 = p->dtype != MOE_DTYPE_F32;  // the dtype of x: bf16 for the bf16 and MXFP8 layers
  ep->out_bf16 = 0;
  if (epi) {
    if (epi->out_dtype != MOE_DTYPE_F32 && epi->out_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    ep->out_bf16 = epi->out_dtype == MOE_DTYPE_BF16;
    ep->residual = epi->residual;
    if (epi->residual && ((uintptr_t)epi->residual % 16)) return MOE_ERR_INVALID_ARGUMENT;
  }
  if ((uintptr_t)out % 16) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ------------------------------------------------------ debug validation --
// MOE_DEBUG_VALIDATE=1 in the environment: before launching anything, each
// entry point copies the device-resident inputs it trusts to the host
// (synchronising the stream) and checks them: logits finite, topk_idx in
// [0, E), src_block in [0, S), offsets starting at 0, non-decreasing and
// ending at most at R, flat_to_sorted in [-1, R).  A failed check returns
// MOE_ERR_INVALID_ARGUMENT and launches nothing.  Host memory only; for
// debugging, not for timed runs.
bool debug_validate() {
  const char* v = getenv("MOE_DEBUG_VALIDATE");
  return v && v[0] == '1' && v[1] == 0;
}

// MOE_DEBUG_SHUFFLE=<n>: the seed of the reordering check (0 or unset: the
// usual order; anything but a decimal number below 2^32 counts as unset).
uint32_t debug_shuffle() {
  const char* v = getenv("MOE_DEBUG_SHUFFLE");
  if (!v || !*v) return 0;
  uint64_t n = 0;
  for (const char* c = v; *c; ++c) {
    if (*c < '0' || *c > '9') return 0;
    n = n * 10 + (uint64_t)(*c - '0');
    if (n > 0xffffffffull) return 0;
  }
  return (uint32_t)n;
}

template <typename T>
bool fetch(std::vector<T>& h, const T* d, int64_t n, hipStream_t s) {
  h.resize(n > 0 ? (size_t)n : 0);
  if (n <= 0) return true;
  if (hipMemcpyAsync(h.data(), d, (size_t)n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess) return false;
  return hipStreamSynchronize(s) == hipSuccess;
}

moe_status_t check_range(const int32_t* d, int64_t n, int32_t lo, int32_t hi, hipStream_t s) {
  std::vector<int32_t> h;
  if (!fetch(h, d, n, s)) return MOE_ERR_HIP;
  for (int32_t v : h)
    if (v < lo || v >= hi) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_status_t validate_logits(const moe_problem_t* p, const float* logits, hipStream_t s) {
  std::vector<float> h;
  if (!fetch(h, logits, p->num_tokens * (int64_t)p->num_experts, s)) return MOE_ERR_HIP;
  for (float v : h)
    if (!isfinite(v)) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_status_t validate_routing(const moe_problem_t* p, const int32_t* topk_idx, const int32_t* src_block,
                              hipStream_t s) {
  moe_status_t st = check_range(topk_idx, p->num_tokens * (int64_t)p->topk, 0, p->num_experts, s);
  if (st == MOE_OK && p->num_src_blocks > 1) st = check_range(src_block, p->num_tokens, 0, p->num_src_blocks, s);
  return st;
}

moe_status_t validate_offsets(const moe_problem_t* p, const int32_t* offsets, hipStream_t s) {
  std::vector<int32_t> h;
  const int G = segments(p);
  if (!fetch(h, offsets, G + 1, s)) return MOE_ERR_HIP;
  if (h[0] != 0) return MOE_ERR_INVALID_ARGUMENT;
  for (int g = 0; g < G; ++g)
    if (h[g + 1] < h[g]) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)h[G] > p->num_tokens * p->topk) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// ------------------------------------------------------------ dispatch ---
// Argument checks of moe_dispatch and its allocation-free variant.
moe_status_t check_dispatch(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                            const int32_t* src_block, const int32_t* counts, const int32_t* offsets,
                            const int32_t* sorted_to_flat, const int32_t* flat_to_sorted, const void* x_perm) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (p->num_src_blocks > 1 && !src_block && p->num_tokens > 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->num_tokens > 0) {
    if (!x || !topk_idx || !sorted_to_flat || !flat_to_sorted || !x_perm) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || !aligned(x_perm, 16)) return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

// Bookkeeping and copy of the dispatch with the scratch `ws` (already sized).
moe_status_t dispatch_launch(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                             const int32_t* src_block, int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat,
                             int32_t* flat_to_sorted, void* x_perm, void* ws, hipStream_t s) {
  if (debug_validate() && p->num_tokens > 0) {
    const moe_status_t st = validate_routing(p, topk_idx, src_block, s);
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_dispatch(plan_of(p), topk_idx, p->num_src_blocks > 1 ? src_block : nullptr, counts,
                                    offsets, sorted_to_flat, flat_to_sorted, x, (int64_t)p->hidden * elem_bytes(p),
                                    x_perm, (int32_t*)ws, s));
}

// Workspace of the whole layer, carved in this order (each region 256-B aligned).
struct LayerWs {
  size_t status, topk_idx, topk_w, counts, offsets, s2f, f2s, perm, x_perm, hact, y, fused, gemm, total;
};

LayerWs layer_ws(const moe_problem_t* p) {
  const int64_t M = p->num_tokens, R = M * p->topk;
  const int G = segments(p);
  const size_t eb = elem_bytes(p);
  const PermutePlan pl = plan_of(p);
  LayerWs w;
  size_t o = 0;
  w.status = o; o += align_up(kAlign);
  w.topk_idx = o; o += align_up((size_t)R * 4);
  w.topk_w = o; o += align_up((size_t)R * 4);
  w.counts = o; o += align_up((size_t)G * 4);
  w.offsets = o; o += align_up((size_t)(G + 1) * 4);
  w.s2f = o; o += align_up((size_t)R * 4);
  w.f2s = o; o += align_up((size_t)R * 4);
  w.perm = o; o += align_up(permute_ws_bytes(pl));
  w.x_perm = o; o += align_up((size_t)R * p->hidden * eb);
  w.hact = o; o += align_up(hact_bytes(p, R));
  w.y = o; o += align_up((size_t)R * p->hidden * 4);
  w.fused = o; o += align_up(fused_ws_bytes(p->num_tokens, p->hidden, p->ffn, held(p), p->topk,
                                             p->num_src_blocks));
  w.gemm = o; o += align_up(p->dtype == MOE_DTYPE_BF16 ? gemm_split_ws_bytes() : 0);  // MXFP8 does not split
  w.total = o;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return (2 << 16) | 0; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE_TIMEOUT: return "MOE_ERR_DEVICE_TIMEOUT";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(const moe_problem_t* p, int32_t op) {
  if (check_problem(p) != MOE_OK) return 0;
  switch (op) {
    case MOE_OP_DISPATCH: return permute_ws_bytes(plan_of(p));
    case MOE_OP_GROUPED_GEMM: return p->dtype == MOE_DTYPE_BF16 ? gemm_split_ws_bytes() : 0;
    case MOE_OP_LAYER: return layer_ws(p).total;
  }
  return 0;
}

moe_status_t moe_route(const moe_problem_t* p, const float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->num_tokens == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (debug_validate()) {
    st = validate_logits(p, logits, (hipStream_t)stream);
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_route(logits, p->num_tokens, p->num_experts, p->topk, topk_idx, topk_w,
                                 (hipStream_t)stream));
}

moe_status_t moe_dispatch(const moe_problem_t* p, const void* x, const int32_t* topk_idx, const int32_t* src_block,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                          void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_dispatch(p, x, topk_idx, src_block, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm);
  if (st != MOE_OK) return st;
  if (ws_bytes < permute_ws_bytes(plan_of(p)) || !ws) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return dispatch_launch(p, x, topk_idx, src_block, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm, ws,
                         (hipStream_t)stream);
}

moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                                  const int32_t* src_block, int32_t* counts, int32_t* offsets,
                                  int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_perm, void* stream) {
  moe_status_t st = check_dispatch(p, x, topk_idx, src_block, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm);
  if (st != MOE_OK) return st;
  if (permute_ws_bytes(plan_of(p)) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* scratch_addr = nullptr;
  if (static_scratch(&scratch_addr) != hipSuccess) return MOE_ERR_HIP;
  return dispatch_launch(p, x, topk_idx, src_block, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm,
                         scratch_addr, (hipStream_t)stream);
}

moe_status_t moe_grouped_gemm(const moe_problem_t* p, int32_t layer, const void* a, const void* w0, const void* w1,
                              const int32_t* offsets, void* c, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (layer != 0 && layer != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!offsets || !w0 || (layer == 0 && !w1)) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t R = p->num_tokens * p->topk;
  if (R > 0 && (!a || !c)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(a, 16) || !aligned(c, 16) || !aligned(w0, 16) || (layer == 0 && !aligned(w1, 16)))
    return MOE_ERR_INVALID_ARGUMENT;
  GemmProblem gp;
  gp.layer = layer;
  gp.a = a;
  gp.w0 = w0;
  gp.w1 = layer == 0 ? w1 : nullptr;
  gp.offsets = offsets;
  gp.c = c;
  gp.R = R;
  gp.K = layer == 0 ? p->hidden : p->ffn;
  gp.N = layer == 0 ? p->ffn : p->hidden;
  gp.E = held(p);
  gp.G = segments(p);
  // a workspace smaller than moe_workspace_bytes(p, MOE_OP_GROUPED_GEMM)
  // (or none) only disables the split of the last round
  if (ws && !aligned(ws, 16)) return MOE_ERR_INVALID_ARGUMENT;
  gp.ws = ws;
  gp.ws_bytes = ws ? ws_bytes : 0;
  gp.rowmap = combine_blocks(p);
  gp.shuffle = debug_shuffle();
  hipStream_t s = (hipStream_t)stream;
  if (debug_validate()) {
    st = validate_offsets(p, offsets, s);
    if (st != MOE_OK) return st;
  }
  if (is_mx(p)) return hip_status(launch_grouped_gemm_mx(gp, s));
  return hip_status(p->dtype == MOE_DTYPE_BF16 ? launch_grouped_gemm_bf16(gp, s) : launch_grouped_gemm_f32(gp, s));
}

moe_status_t moe_combine_ex(const moe_problem_t* p, const float* y, const float* topk_w,
                            const int32_t* flat_to_sorted, const moe_epilogue_t* epi, void* out, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->num_tokens == 0) return MOE_OK;
  if (!y || !topk_w || !flat_to_sorted || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(y, 16) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARGUMENT;
  OutEpilogue ep;
  st = epilogue_of(p, epi, out, &ep);
  if (st != MOE_OK) return st;
  if (debug_validate()) {
    st = check_range(flat_to_sorted, p->num_tokens * (int64_t)p->topk, -1, (int32_t)(p->num_tokens * p->topk),
                     (hipStream_t)stream);
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_combine(y, topk_w, flat_to_sorted, p->num_tokens, p->hidden, p->topk, ep,
                                   (hipStream_t)stream));
}

moe_status_t moe_combine(const moe_problem_t* p, const float* y, const float* topk_w, const int32_t* flat_to_sorted,
                         float* out, void* stream) {
  return moe_combine_ex(p, y, topk_w, flat_to_sorted, nullptr, out, stream);
}

int32_t moe_layer_default_movers(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK || p->dtype != MOE_DTYPE_BF16) return -1;
  return fused_default_movers(p->num_tokens, p->hidden, p->ffn, p->num_experts, p->topk, p->num_src_blocks,
                              held(p), p->dtype, device_cu_count());
}

moe_status_t moe_layer_ex(const moe_problem_t* p, const void* x, const float* logits, const int32_t* src_block,
                          const void* w_gate, const void* w_up, const void* w_down, const moe_epilogue_t* epi,
                          void* out, const moe_layer_aux_t* aux, const moe_layer_opts_t* opts, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const int64_t M = p->num_tokens;
  if (!w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && (!x || !logits || !out)) return MOE_ERR_INVALID_ARGUMENT;
  if (p->num_src_blocks > 1 && !src_block && M > 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  OutEpilogue ep;
  st = epilogue_of(p, epi, out, &ep);
  if (st != MOE_OK) return st;
  const LayerWs L = layer_ws(p);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, kAlign)) return MOE_ERR_INVALID_ARGUMENT;
  moe_layer_aux_t a;
  memset(&a, 0, sizeof a);
  if (aux) a = *aux;
  if (a.x_perm && !aligned(a.x_perm, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (a.hact && !aligned(a.hact, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (a.y && !aligned(a.y, 16)) return MOE_ERR_INVALID_ARGUMENT;
  const int G = segments(p);
  int32_t* idx = a.topk_idx ? a.topk_idx : at<int32_t>(ws, L.topk_idx);
  float* w = a.topk_w ? a.topk_w : at<float>(ws, L.topk_w);
  int32_t* counts = a.counts ? a.counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = a.offsets ? a.offsets : at<int32_t>(ws, L.offsets);
  int32_t* s2f = a.sorted_to_flat ? a.sorted_to_flat : at<int32_t>(ws, L.s2f);
  int32_t* f2s = a.flat_to_sorted ? a.flat_to_sorted : at<int32_t>(ws, L.f2s);
  void* xp = a.x_perm ? a.x_perm : at<void>(ws, L.x_perm);
  void* hact = a.hact ? a.hact : at<void>(ws, L.hact);
  float* y = a.y ? a.y : at<float>(ws, L.y);
  int32_t* status = at<int32_t>(ws, L.status);
  const int32_t* src = p->num_src_blocks > 1 ? src_block : nullptr;
  hipStream_t s = (hipStream_t)stream;

  moe_layer_opts_t o;
  o.n_mover = -1;
  o.grid = 0;
  o.fused = 1;
  o.spin_limit = 0;
  o.gather = -1;
  if (opts) o = *opts;

  const int cus = device_cu_count();
  // n_mover < 0 asks the profiled table, which may pick the kernel chain
  const int movers = o.n_mover >= 0 ? o.n_mover
                                    : fused_default_movers(M, p->hidden, p->ffn, p->num_experts, p->topk,
                                                           p->num_src_blocks, held(p), p->dtype, cus);
  if (movers == kTableUnusable) return MOE_ERR_INVALID_ARGUMENT;
  if (debug_validate() && M > 0) {
    st = validate_logits(p, (const float*)logits, s);
    if (st == MOE_OK && p->num_src_blocks > 1) st = check_range(src_block, M, 0, p->num_src_blocks, s);
    if (st != MOE_OK) return st;
  }
  // zeroed by kernels rather than memset nodes, so that the call can be
  // captured into a HIP graph
  hipError_t e;
  if (M == 0) {
    // nothing routed: counts and offsets are all zero
    e = launch_fill_i32(status, 1, 0, s);
    if (e == hipSuccess) e = launch_fill_i32(counts, G, 0, s);
    if (e == hipSuccess) e = launch_fill_i32(offsets, G + 1, 0, s);
    return hip_status(e);
  }
  const bool fused = o.fused != 0 && p->dtype == MOE_DTYPE_BF16 && movers >= 0;
  // Layer0 of the fused kernel gathers its token rows from x unless the
  // caller asks for the X_perm copy (o.gather == 0)
  const bool gather = o.gather != 0;
  FusedArgs fa;
  if (fused) {
    fa.M = M;
    fa.H = p->hidden;
    fa.F = p->ffn;
    fa.E = held(p);
    fa.k = p->topk;
    fa.G = G;
    fa.x = x;
    fa.x_perm = gather ? nullptr : xp;
    fa.w_gate = w_gate;
    fa.w_up = w_up;
    fa.w_down = w_down;
    fa.topk_w = w;
    fa.offsets = offsets;
    fa.s2f = s2f;
    fa.f2s = f2s;
    fa.hact = hact;
    fa.y = y;
    fa.out = ep;
    fa.status = status;
    fa.flags = at<int32_t>(ws, L.fused);
    fa.mt_max = fused_mt_max(M, p->hidden, p->topk, G);
    fa.grid = o.grid > 0 ? o.grid : cus;
    fa.n_mover = movers;
    fa.spin_limit = o.spin_limit;
    fa.shuffle = debug_shuffle();
    // checked before anything is launched
    const moe_status_t fs = fused_check(fa, cus);
    if (fs != MOE_OK) return fs;
  }
  // the route kernel also clears the status word and (fused) the ready counters
  e = launch_route(logits, M, p->num_experts, p->topk, idx, w, s, status, 1, fused ? fa.flags : nullptr,
                   fused ? fused_flag_words(M, p->hidden, p->topk, G) : 0);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (fused) {
    // gathering, the kernel reads token rows straight from x and X_perm is
    // produced only when the caller asks for it
    e = launch_dispatch(plan_of(p), idx, src, counts, offsets, s2f, f2s, x, (int64_t)p->hidden * elem_bytes(p),
                        (!gather || a.x_perm) ? xp : nullptr, at<int32_t>(ws, L.perm), s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_fused_layer(fa, s));
  }
  e = launch_dispatch(plan_of(p), idx, src, counts, offsets, s2f, f2s, x, (int64_t)p->hidden * elem_bytes(p), xp,
                      at<int32_t>(ws, L.perm), s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  GemmProblem gp;
  gp.R = M * p->topk;
  gp.E = held(p);
  gp.G = G;
  gp.offsets = offsets;
  gp.layer = 0;
  gp.a = xp;
  gp.w0 = w_gate;
  gp.w1 = w_up;
  gp.c = hact;
  gp.K = p->hidden;
  gp.N = p->ffn;
  gp.ws = at<void>(ws, L.gemm);
  gp.ws_bytes = L.total - L.gemm;
  gp.rowmap = combine_blocks(p);
  gp.shuffle = debug_shuffle();
  e = is_mx(p) ? launch_grouped_gemm_mx(gp, s)
              : (p->dtype == MOE_DTYPE_BF16 ? launch_grouped_gemm_bf16(gp, s) : launch_grouped_gemm_f32(gp, s));
  if (e != hipSuccess) return MOE_ERR_HIP;
  gp.layer = 1;
  gp.a = hact;
  gp.w0 = w_down;
  gp.w1 = nullptr;
  gp.c = y;
  gp.K = p->ffn;
  gp.N = p->hidden;
  e = is_mx(p) ? launch_grouped_gemm_mx(gp, s)
              : (p->dtype == MOE_DTYPE_BF16 ? launch_grouped_gemm_bf16(gp, s) : launch_grouped_gemm_f32(gp, s));
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_combine(y, w, f2s, M, p->hidden, p->topk, ep, s));
}

moe_status_t moe_layer(const moe_problem_t* p, const void* x, const float* logits, const int32_t* src_block,
                       const void* w_gate, const void* w_up, const void* w_down, float* out,
                       const moe_layer_aux_t* aux, const moe_layer_opts_t* opts, void* ws, size_t ws_bytes,
                       void* stream) {
  return moe_layer_ex(p, x, logits, src_block, w_gate, w_up, w_down, nullptr, out, aux, opts, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_mxfp8(int64_t rows, int32_t cols, int32_t src_dtype, const void* src, void* dst,
                                void* stream) {
  if (rows < 0 || cols < 128 || cols % 128) return MOE_ERR_INVALID_ARGUMENT;
  if (src_dtype != MOE_DTYPE_BF16 && src_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (rows == 0) return MOE_OK;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (rows >= (1ll << 40) / cols) return MOE_ERR_UNSUPPORTED;  // rows * cols < 2^40, checked without forming it
  return hip_status(launch_mx_quantize(src, src_dtype == MOE_DTYPE_BF16, rows, cols, dst, (hipStream_t)stream));
}

moe_status_t moe_transpose_weights(int64_t batch, int32_t rows, int32_t cols, int32_t dtype, const void* src,
                                   void* dst, void* stream) {
  if (batch < 0 || rows <= 0 || cols <= 0 || rows % 64 || cols % 64) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (batch == 0) return MOE_OK;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARGUMENT;
  // sizes bounded before any product that could wrap: batch * rows * cols < 2^40
  const uint64_t elems = (uint64_t)rows * (uint64_t)cols;  // < 2^62
  if (elems >= (1ull << 40) || (uint64_t)batch >= (1ull << 40) / elems) return MOE_ERR_UNSUPPORTED;
  const uint64_t bytes = (uint64_t)batch * elems * (dtype == MOE_DTYPE_BF16 ? 2u : 4u);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARGUMENT;  // overlapping buffers
  return hip_status(launch_transpose(src, dst, batch, rows, cols, dtype == MOE_DTYPE_BF16, (hipStream_t)stream));
}

moe_status_t moe_debug_device_status(const moe_problem_t* p, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const LayerWs L = layer_ws(p);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  int32_t v = 0;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&v, at<int32_t>(ws, L.status), sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  return v == 0 ? MOE_OK : (moe_status_t)v;
}

}  // extern "C"

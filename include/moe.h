/*
 * moe.h -- C ABI of the MoE layer hot path on AMD Instinct MI355X (gfx950).
 *
 * One MoE layer, in the order the pages state it:
 *   route     top-k expert choice per token and renormalised weights
 *   dispatch  count rows per (source block, expert), prefix-sum offsets,
 *             stable permutation, gather of token rows sorted by segment
 *   grouped   Layer0: gate/up products + SwiGLU; Layer1: down product,
 *   GEMM      both as one grouped GEMM over all experts
 *   combine   top-k weighted reduction of each token's expert outputs,
 *             optionally plus a residual and cast to bf16 (epilogue)
 *   layer     all of the above in one persistent kernel: one ordered work
 *             queue of Layer0 tiles, Layer1 tiles and combine items, with
 *             ready counters between them
 *
 * Sources (cited by page and section):
 *   [COMET]  "COMET: Fine-grained Computation-communication Overlapping for
 *            Mixture-of-Experts" (paper review): §3.2 Layer0/Layer1
 *            pipelines; §4.1.1 shared-tensor decomposition (Layer0 along M,
 *            Layer1 along N because of the Top-K reduction); §4.1.2
 *            rescheduling (reorder by source, column-wise GroupGEMM);
 *            §4.2.1 thread-block specialisation; §4.2.2 adaptive
 *            thread-block allocation from profiled metadata.
 *   [GGEMM]  "Grouped GEMM 为什么适合 MoE" (why grouped GEMM suits MoE):
 *            C_i = A_i B_i over G problems, tile queue, double buffering,
 *            L2 locality, fused epilogue (GemmAdd: Y = cast(Acc + Add)).
 *   [PTO]    "PTO MoE算子实战" (PTO MoE operator article): the seven serial
 *            stages (reorder, AllToAll, reorder, GMM1/SwiGLU/GMM2, reorder,
 *            AllToAllV, top-K weighted accumulation); MegaMoE fusion;
 *            count-as-flag.
 *
 * Conventions for every call:
 *   - Tensor arguments are DEVICE pointers to row-major, contiguous memory,
 *     16-byte aligned (except topk/int32 arrays: 4-byte aligned).  The caller
 *     allocates and owns every buffer; the library allocates nothing per call
 *     and keeps no per-call state.
 *   - `stream` is a hipStream_t (passed as void*); NULL means the default
 *     stream.  Every call only enqueues work on `stream` and returns; none
 *     synchronises the device or copies device memory to the host.
 *   - Errors: arguments are checked on the host; a failed check returns a
 *     status and enqueues nothing.  Device-resident inputs are trusted:
 *     logits must be finite, src_block values must lie in [0, S), topk_idx
 *     in [0, E), and offsets must be the exclusive prefix sum of the counts
 *     of the same call sequence.  Violating these gives unspecified results
 *     (the kernels keep every memory access inside the caller's buffers: an
 *     out-of-range expert id or source block makes its pair a dropped one).
 *   - MOE_DEBUG_VALIDATE=1 in the environment makes every entry point check
 *     those device-resident inputs before it launches anything: it copies
 *     them to host memory (synchronising `stream`) and returns
 *     MOE_ERR_INVALID_ARGUMENT if logits are not finite (moe_route,
 *     moe_layer), topk_idx is outside [0, E) or src_block outside [0, S)
 *     (moe_dispatch, moe_layer), offsets do not start at 0, decrease, or
 *     end past R (moe_grouped_gemm), or flat_to_sorted is outside [-1, R)
 *     (moe_combine).  For debugging only: it synchronises and copies.
 *   - MOE_TUNING_TABLE=<path> makes moe_layer's plan (the split table of
 *     the fused layer, used when opts->n_mover < 0) come from that JSON file
 *     instead of the table compiled in (the one stored in
 *     combine_topk_gate_amd/tuning/mi355x.json): {"entries": [{"M": .., "H":
 *     .., "F": .., "E": .., "k": .., "S": .., "EL": .., "n_mover": ..}, ...]}
 *     with n_mover -1 for the kernel chain; other keys are ignored.
 *     combine_topk_gate_amd/tune_split.py --write profiles a GPU and writes
 *     one.  A file that cannot be read or parsed makes moe_layer return
 *     MOE_ERR_INVALID_ARGUMENT (when it needs the plan) and
 *     moe_layer_default_movers return -2; it is read again when the
 *     variable changes.
 *   - MOE_DEBUG_SHUFFLE=<seed> (a decimal number, 0 or unset: off) makes the
 *     grouped GEMMs and the fused layer take their tiles in a seeded
 *     permutation of the usual order: inside the full rounds, and separately
 *     inside a last round that is split along k or halved; in the fused
 *     kernel inside each section of its queue (Layer0 tiles, one chunk's
 *     Layer1 tiles, one chunk's combine items).  Every output element is
 *     computed by one item in a fixed order of its own, so results must be
 *     bit-identical to the usual order ([COMET] §4.1.2: rescheduling does
 *     not change results); a difference is a scheduling bug.  A check, not
 *     a mode: the permuted order loses the tiles' cache locality.
 *   - Symbols: M tokens, H hidden, F expert width, E experts routing
 *     chooses from, EL experts held by the call (local_experts, = E unless
 *     set), k = topk, S source blocks, G = S*EL segments, R = M*k routed
 *     pairs (the capacity of every per-pair buffer).
 *   - Weight storage: W_gate, W_up stored [EL,F,H] and W_down stored
 *     [EL,H,F]: row f of W_gate[e] is column f of the H x F matrix of the
 *     math (x W_gate), so every stored row is contiguous in the reduction
 *     index.  Weight slot l holds expert expert_base + l.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment */
  MOE_ERR_UNSUPPORTED = 2,      /* valid but outside what the kernels handle */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4,              /* a HIP runtime call failed (launch error) */
  MOE_ERR_DEVICE_TIMEOUT = 5    /* a bounded device wait ran out (fused layer) */
} moe_status_t;

/* MOE_DTYPE_BF16_MXFP8: x, W_gate, W_up and X_perm bf16; the activation
 * Hact and W_down in MXFP8 ([PTO] two-stage SwiGLU: the activation is
 * quantised as SwiGLU produces it).  MXFP8 is the OCP microscaling format
 * with e4m3 elements: per 32 consecutive values of a row one scale byte
 * s, value = e4m3(code) * 2^(s - 127); the scale is 2^X with X =
 * floor(log2 of the block's largest magnitude) - 8 (or s = 0 for an
 * all-zero block), codes are the nearest e4m3 value (ties to even),
 * magnitudes past 448 become 448.  An MXFP8 tensor of rows x cols (cols a
 * multiple of 128) is ONE buffer: rows*cols codes (row-major), then the
 * scale bytes in groups of 32 rows (rows padded to a multiple of 32): the
 * byte of row r, block b (columns 32b .. 32b+31) sits at
 *   (r / 32) * cols + (b / 4) * 128 + (r % 32) * 4 + b % 4,
 * so per group and 128-column quad the 4 bytes of each row lie together.
 * Buffer size: rows*cols + ceil(rows/32)*32*cols/32 bytes.  No reader
 * uses the padding rows' bytes; moe_quantize_mxfp8 writes them as 0,
 * layer 0 leaves them as they are. */
typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1, MOE_DTYPE_BF16_MXFP8 = 2 } moe_dtype_t;

/* Operation whose workspace moe_workspace_bytes sizes. */
typedef enum { MOE_OP_DISPATCH = 0, MOE_OP_GROUPED_GEMM = 1, MOE_OP_LAYER = 2 } moe_op_t;

/*
 * Problem shape.  Limits: 0 <= M, M*k < 2^31; H and F multiples of 64 in
 * [64, 65536]; 1 <= E <= 512; 1 <= k <= min(E, 16); S >= 1; S*EL <= 1024
 * (S*EL <= 1023 when EL < E); R*max(H,F) < 2^31 (32-bit element offsets
 * into the per-pair buffers) and EL*H*F < 2^37 (weights are addressed per
 * expert with 64-bit offsets; the MXFP8 weight scales are one range of
 * EL*H*F/32 bytes).  Beyond these, MOE_ERR_UNSUPPORTED.
 * dtype is the type of x, the weights, X_perm and Hact: MOE_DTYPE_BF16
 * (fp32 accumulation), MOE_DTYPE_F32, or MOE_DTYPE_BF16_MXFP8 (Hact and
 * W_down MXFP8, the rest bf16; F a multiple of 128).  Logits, weights of the top-k and Y
 * are always f32; out is f32 unless an epilogue asks for bf16.
 *
 * Local experts ([COMET] §4.1.2 tokens grouped by source and expert for
 * expert parallelism; [PTO] measured case: 16 local experts per card, the
 * rest on other cards): routing chooses among all E experts; a call with
 * local_experts = EL > 0 holds experts [expert_base, expert_base + EL) and
 * keeps only the pairs routed to them.  Kept pair f goes to segment
 * src * EL + (expert - expert_base); the other pairs are dropped, and the
 * combine's out is this call's share of each token's sum (the partial
 * combine that the holders of the other experts complete).  local_experts =
 * 0 (or E with expert_base 0) is the plain layer.
 */
typedef struct {
  int64_t num_tokens;     /* M */
  int32_t hidden;         /* H */
  int32_t ffn;            /* F */
  int32_t num_experts;    /* E: experts routing chooses from */
  int32_t topk;           /* k */
  int32_t num_src_blocks; /* S (1 unless rows arrive tagged by source block) */
  int32_t dtype;          /* moe_dtype_t */
  int32_t expert_base;    /* first expert held (0 unless local_experts > 0) */
  int32_t local_experts;  /* EL: experts held, expert_base + EL <= E; 0 = all E */
} moe_problem_t;

/* Bytes of device workspace `op` needs for this problem (0 if none).
 * Returns 0 and sets nothing for an invalid problem; check with the call. */
size_t moe_workspace_bytes(const moe_problem_t* p, int32_t op);

/*
 * Route ([COMET] §4.1.1 Top-K reduction; [PTO] seven stages, top-K weighted
 * accumulation).  For each token t: topk_idx[t, 0..k-1] = the k experts with
 * the largest logits[t, :], in descending order of logit; equal logits go to
 * the lower expert index (IEEE comparison: -0.0 ties +0.0).
 * topk_w[t, j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), summed in slot
 * order (softmax over the chosen logits, f32 arithmetic, full-precision exp).
 *   logits   [M,E] f32 (finite), read only
 *   topk_idx [M,k] int32, written
 *   topk_w   [M,k] f32, written
 */
moe_status_t moe_route(const moe_problem_t* p, const float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Dispatch ([PTO] local reorder by expert + count-as-flag counts; [COMET]
 * §4.1.2 reorder by source; §3.2 Layer0 dispatch).  Pair f = t*k + j belongs
 * to segment g = src_block[t]*EL + (topk_idx[t,j] - expert_base) if that
 * expert is held, else it is dropped (src_block NULL means S = 1).
 *   counts[g]          number of pairs in segment g                 [G] int32
 *   offsets            exclusive prefix sum of counts; offsets[G] = the
 *                      number of kept pairs (R when all are held)   [G+1] int32
 *   sorted_to_flat[r]  the pair at sorted position r: segments in order,
 *                      increasing f inside a segment (stable); -1 for
 *                      r >= offsets[G]                              [R] int32
 *   flat_to_sorted     the inverse permutation; -1 for a dropped pair [R] int32
 *   x_perm[r, :]       = x[sorted_to_flat[r] / k, :]  (byte copy) for
 *                      r < offsets[G]; later rows are not written   [R,H] dtype
 *   x                  [M,H] dtype, read only
 * Results are bit-exact and independent of scheduling (no atomics decide
 * an order).  ws must hold moe_workspace_bytes(p, MOE_OP_DISPATCH) bytes.
 */
moe_status_t moe_dispatch(const moe_problem_t* p, const void* x, const int32_t* topk_idx, const int32_t* src_block,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                          void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free dispatch, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): moe_dispatch without the workspace argument.  Its scratch
 * (the per-chunk segment histograms and their prefix sums) is a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends; the call allocates nothing, and
 * the kernels overwrite every scratch word they read, so nothing needs
 * clearing between calls.  Problems whose dispatch workspace
 * (moe_workspace_bytes(p, MOE_OP_DISPATCH)) exceeds that size return
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  All calls on one GPU
 * share its scratch: calls that may run at the same time on one GPU (on
 * different streams, or from different threads without ordering) race and
 * must not be issued; calls ordered on one stream are fine.  Arguments,
 * results and errors are otherwise those of moe_dispatch, bit for bit.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (1u << 20)
moe_status_t moe_dispatch_noalloc(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                                  const int32_t* src_block, int32_t* counts, int32_t* offsets,
                                  int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_perm, void* stream);

/*
 * Grouped GEMM over the G segments ([GGEMM] C_i = A_i B_i with per-problem
 * sizes; segment g uses weight slot g % EL and rows offsets[g] ..
 * offsets[g+1]-1; rows from offsets[G] on are neither read nor written).
 *   layer 0 ([COMET] §3.2 Layer0; [PTO] GMM1 -> SwiGLU):
 *     a  = X_perm [R,H] dtype; w0 = W_gate [EL,F,H]; w1 = W_up [EL,F,H]
 *     c  = Hact [R,F] dtype: Hact[r,f] = silu(g) * u rounded to dtype, where
 *          g = sum_h X_perm[r,h] W_gate[e,f,h], u likewise with W_up, both
 *          accumulated in f32, silu(z) = z / (1 + exp(-z)).
 *   layer 1 ([COMET] §3.2 Layer1; [PTO] GMM2):
 *     a  = Hact [R,F] dtype; w0 = W_down [EL,H,F]; w1 = NULL
 *     c  = Y [R,H] f32: Y[r,n] = sum_f Hact[r,f] W_down[e,n,f], f32 accumulation.
 *   MOE_DTYPE_BF16_MXFP8: layer 0 writes c as an MXFP8 buffer of R x F
 *   (the codes decided on the f32 value silu(g) * u), layer 1 reads a (R x
 *   F) and w0 (EL*H x F) as MXFP8 buffers; the matrix cores multiply the
 *   codes and apply both block scales, accumulating in f32.  No workspace.
 *   offsets [G+1] int32 as produced by moe_dispatch.  Rows of empty segments
 *   produce nothing.
 *   ws (bf16 layers): NULL, or at least moe_workspace_bytes(p,
 *   MOE_OP_GROUPED_GEMM) bytes, 16-byte aligned (a misaligned ws returns
 *   MOE_ERR_INVALID_ARGUMENT).  Layer 1 with it computes the tiles of the
 *   persistent grid's last round in up to 8 ranges of k ([GGEMM] tile
 *   scheduling over uneven problems) whose f32 partial sums a second pass
 *   adds in increasing k order, so the last round ends sooner; without it
 *   (or when smaller), and always in layer 0, those tiles are cut into half
 *   tiles instead.  Every product is still accumulated in f32; only the
 *   grouping of the k sum of those tiles differs, and a given device always
 *   splits the same tiles.  f32 layers use no workspace.
 */
moe_status_t moe_grouped_gemm(const moe_problem_t* p, int32_t layer, const void* a, const void* w0, const void* w1,
                              const int32_t* offsets, void* c, void* ws, size_t ws_bytes, void* stream);

/*
 * Combine ([COMET] §4.1.1/§4.1.2 Top-K reduction, column-wise; [PTO] Combine
 * + Unpermute, top-K weighted accumulation).
 *   out[t, n] = sum_{j=0..k-1} topk_w[t,j] * y[flat_to_sorted[t*k+j], n],
 *   f32, accumulated from zero in slot order j = 0..k-1 (fused multiply-add);
 *   slots whose flat_to_sorted is -1 (pairs of experts not held) are left
 *   out, so a token with none of them gets 0.
 *   y [R,H] f32; topk_w [M,k] f32; flat_to_sorted [R] int32; out [M,H] f32.
 */
moe_status_t moe_combine(const moe_problem_t* p, const float* y, const float* topk_w, const int32_t* flat_to_sorted,
                         float* out, void* stream);

/*
 * Output epilogue of the combine ([GGEMM] fused GemmAdd epilogue, Y =
 * cast(Acc + Add)): acc is the combine's f32 sum above; then
 *   out[t, n] = cast(acc[t, n] + residual[t, n])
 * with one f32 addition (no residual: acc itself) and the cast to out_dtype:
 * f32 keeps the value, bf16 rounds to nearest even.
 *   residual  [M,H] in the dtype of x (f32 for f32 layers, else bf16), or NULL
 *   out_dtype MOE_DTYPE_F32 or MOE_DTYPE_BF16
 */
typedef struct {
  const void* residual;
  int32_t out_dtype;
} moe_epilogue_t;

/* moe_combine with an epilogue (NULL epi: as moe_combine); out [M,H] in
 * epi->out_dtype, 16-byte aligned; residual 16-byte aligned. */
moe_status_t moe_combine_ex(const moe_problem_t* p, const float* y, const float* topk_w,
                            const int32_t* flat_to_sorted, const moe_epilogue_t* epi, void* out, void* stream);

/* Optional device buffers that receive moe_layer's intermediates (any field
 * may be NULL, then the workspace holds that intermediate). */
typedef struct {
  int32_t* topk_idx;       /* [M,k] */
  float* topk_w;           /* [M,k] */
  int32_t* counts;         /* [G] */
  int32_t* offsets;        /* [G+1] */
  int32_t* sorted_to_flat; /* [R] */
  int32_t* flat_to_sorted; /* [R] */
  void* x_perm;            /* [R,H] dtype */
  void* hact;              /* [R,F] dtype */
  float* y;                /* [R,H] f32 */
} moe_layer_aux_t;

/* Schedule options of the fused layer (NULL = defaults).  Results do not
 * depend on them: every output element is computed in a fixed order. */
typedef struct {
  int32_t n_mover;     /* dedicated combine workgroups; 0: combine items share the work queue;
                          <0: the profiled split table's plan (which may be the chain) */
  int32_t grid;        /* total persistent workgroups; <=0: every CU, one each */
  int32_t fused;       /* 0: run the unfused kernel chain instead of the fused kernel */
  int32_t spin_limit;  /* >0: bound on each device wait (polls); 0: default bound */
  int32_t gather;      /* Layer0's token rows in the fused kernel: 1 or <0 (default): read straight
                          from x through sorted_to_flat (X_perm not written unless aux->x_perm is
                          given); 0: the dispatch writes X_perm and Layer0 reads it, as in the chain
                          (measured: 1% faster at Mixtral's shape, 1-2% slower at the others) */
} moe_layer_opts_t;

/*
 * The whole layer ([COMET] §4.2.1 thread-block specialisation, §4.2.2
 * adaptive allocation, §4.1.1-§4.1.2 shared-tensor decomposition and
 * column-wise Layer1; [PTO] MegaMoE seven-stage fusion, ready counters,
 * dynamic core grouping): route, dispatch (the X_perm copy only with
 * opts->gather = 0), then one persistent kernel (bf16 layers) whose
 * workgroups take, from one ordered queue, Layer0 tiles (token rows read
 * straight from x through sorted_to_flat, or from X_perm with gather = 0),
 * Layer1 tiles column chunk by column chunk (each once its row tile's
 * Layer0 tiles are done), and combine items (a column chunk of a block of
 * tokens, once that chunk's Layer1 tiles are done) -- either on n_mover
 * dedicated workgroups or in the shared queue.  Counters in the workspace
 * are the ready flags.  f32 layers, and opts->fused == 0, run the kernel
 * chain moe_route -> moe_dispatch -> moe_grouped_gemm(0) ->
 * moe_grouped_gemm(1) -> moe_combine instead.  The fused kernel gives the
 * same bits as that chain run without a grouped-GEMM workspace; moe_layer's
 * own chain passes one (the last round split along k, see
 * moe_grouped_gemm), which regroups the k sum of those tiles only.
 *   x [M,H] dtype; logits [M,E] f32; src_block [M] int32 or NULL (S = 1);
 *   w_gate, w_up [EL,F,H]; w_down [EL,H,F]; out [M,H] f32 (the partial
 *   combine when EL < E).
 *   aux: gathering, the fused path writes X_perm only if aux->x_perm is
 *   given.
 * The fused kernel needs its whole grid resident (one workgroup per CU):
 * opts->grid above that returns MOE_ERR_UNSUPPORTED; n_mover >= grid returns
 * MOE_ERR_INVALID_ARGUMENT.  Residency is checked against the device, not
 * against other work: a fused call running beside other kernels that hold
 * CUs (another stream, another fused call) can have workgroups wait for
 * ones that cannot start, until the bounded waits end it with
 * MOE_ERR_DEVICE_TIMEOUT.  Run the fused path alone on the device, or with
 * opts->grid at most the CUs it may have; the kernel chain has no such
 * requirement.  If a bounded device wait runs out, the kernel
 * stops early and records MOE_ERR_DEVICE_TIMEOUT in the workspace; read it
 * with moe_debug_device_status.
 */
moe_status_t moe_layer(const moe_problem_t* p, const void* x, const float* logits, const int32_t* src_block,
                       const void* w_gate, const void* w_up, const void* w_down, float* out,
                       const moe_layer_aux_t* aux, const moe_layer_opts_t* opts, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * MXFP8 quantisation (the format of MOE_DTYPE_BF16_MXFP8) of rows x cols
 * values, blocks of 32 along a row: src [rows, cols] bf16 (src_dtype
 * MOE_DTYPE_BF16) or f32; dst one MXFP8 buffer of rows*cols +
 * ceil(rows/32)*32*cols/32 bytes (codes, then scales in the grouped order
 * above).  cols a multiple of 128 (else MOE_ERR_INVALID_ARGUMENT); src and
 * dst 16-byte aligned.  For W_down, rows = EL*H and cols = F.
 */
moe_status_t moe_quantize_mxfp8(int64_t rows, int32_t cols, int32_t src_dtype, const void* src, void* dst,
                                void* stream);

/*
 * Weight preparation for callers holding the weight matrices as the math
 * writes them (reading of the pages' layer: x·W_gate with W_gate of H x F,
 * h·W_down with W_down of F x H): a batched transpose src [batch, rows,
 * cols] -> dst [batch, cols, rows] that gives the storage the layer reads
 * (W_gate, W_up: batch = EL, rows = H, cols = F -> [EL,F,H]; W_down: rows =
 * F, cols = H -> [EL,H,F]).  dtype MOE_DTYPE_BF16 or MOE_DTYPE_F32 (for an
 * MXFP8 layer, transpose the bf16 W_down, then moe_quantize_mxfp8 it).
 * rows and cols multiples of 64, src and dst 16-byte aligned and not
 * overlapping (else MOE_ERR_INVALID_ARGUMENT).  Enqueued on stream; meant
 * to run once, before the layer calls, not on the hot path.
 */
moe_status_t moe_transpose_weights(int64_t batch, int32_t rows, int32_t cols, int32_t dtype, const void* src,
                                   void* dst, void* stream);

/* moe_layer with the combine's epilogue (NULL epi: as moe_layer); out [M,H]
 * in epi->out_dtype.  The fused kernel and the chain apply it in the same
 * f32 order, so they still agree bit for bit. */
moe_status_t moe_layer_ex(const moe_problem_t* p, const void* x, const float* logits, const int32_t* src_block,
                          const void* w_gate, const void* w_up, const void* w_down, const moe_epilogue_t* epi,
                          void* out, const moe_layer_aux_t* aux, const moe_layer_opts_t* opts, void* ws,
                          size_t ws_bytes, void* stream);

/* The plan the profiled split table picks for this problem (what moe_layer
 * does when opts->n_mover < 0): the number of dedicated combine workgroups
 * of the fused kernel (0: the combine shares the work queue), or -1 when the
 * layer runs as the kernel chain (f32 and MXFP8 layers, shapes where
 * profiling found the chain faster, and shapes the table does not list:
 * on MI355X the chain was faster on every shape measured) or the problem
 * is invalid; -2 when MOE_TUNING_TABLE names a file that cannot be read or
 * parsed. */
int32_t moe_layer_default_movers(const moe_problem_t* p);

/* Synchronises `stream` and returns the device status the last moe_layer
 * on this workspace recorded (MOE_OK or MOE_ERR_DEVICE_TIMEOUT).  Tests only. */
moe_status_t moe_debug_device_status(const moe_problem_t* p, void* ws, size_t ws_bytes, void* stream);

/* Human-readable name of a status. */
const char* moe_status_string(moe_status_t s);

/* ABI version: (major << 16) | minor. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */

/*
 * moe_oracle.c -- plain, slow CPU oracle for the MoE layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (one MoE layer, the plain definition, in fp64):
 *   route    -> per token the k largest gate logits, descending, ties to the
 *               lower expert index; weights = softmax over the k chosen
 *               logits.  ("topK weighted accumulation", PTO MoE article,
 *               section on the seven serial stages; COMET review §4.1.1
 *               names the Top-K reduction that couples rows along M.)
 *   segments -> counts per (source block, expert) and their exclusive
 *               prefix sum (PTO MoE article, "count-as-flag": the per-expert
 *               row counts).
 *   permute  -> pairs f = t*k + j listed segment by segment, increasing f
 *               inside a segment (local reorder by expert, PTO MoE article,
 *               seven serial stages; reorder by source first, COMET review
 *               §4.1.2 "Layer0" rescheduling).
 *   dispatch -> X_perm[r] = x[token of sorted_to_flat[r]] (COMET review §3.2,
 *               Layer0 dispatch).
 *   layer 0  -> g = X_r W_gate[e], u = X_r W_up[e], h = silu(g) * u (SwiGLU,
 *               PTO MoE article "GMM1 -> SwiGLU"); for bf16 layers h is
 *               rounded to bf16 (round to nearest even) because it is the
 *               bf16 activation the down projection consumes.
 *   layer 1  -> Y_r = h W_down[e], kept in fp64 (COMET review §3.2, Layer1).
 *   combine  -> out[t] = sum_j w[t,j] * Y[flat_to_sorted[t*k+j]], summed from
 *               zero in slot order j = 0..k-1 (COMET review §4.1.1 Top-K
 *               reduction; PTO MoE article "Combine / Unpermute").
 *   fp8 act  -> optionally the activation is quantised as SwiGLU produces it
 *               (PTO MoE article, two-stage SwiGLU: each segment consumed
 *               and quantised at once) and the down product runs on the
 *               quantised values.  The format is the open OCP microscaling
 *               one, MXFP8 with e4m3 elements: blocks of 32 values along F
 *               share a power-of-two scale; W_down is given in the same
 *               format (see the fp8 section below).
 *   epilogue -> out = cast(acc + residual) (grouped-GEMM article, fused
 *               GemmAdd epilogue: the accumulator plus an added tensor,
 *               then the cast to the output type), bf16 by round to
 *               nearest even.
 *
 * Local experts (expert parallelism, COMET review §4.1.2 and the PTO MoE
 * article's measured case of 16 local experts per card): routing chooses
 * among all E experts, and a call that holds only experts
 * [base, base + EL) keeps the pairs routed to them.  Kept pair f goes to
 * segment src * EL + (expert - base); the other pairs are dropped: they get
 * no sorted position (flat_to_sorted[f] = -1), sorted positions past the
 * kept ones hold -1, and the combine leaves them out, so out is this
 * call's share of the token's sum (the partial combine that the other
 * holders of experts complete).  EL = E, base = 0 is the plain layer.
 *
 * Storage conventions (shared with the library's public header by
 * specification only, not by code):
 *   logits  [M,E] f32, x [M,H] (f32 or bf16 bits), src_block [M] i32 or NULL
 *   W_gate, W_up stored [E,F,H] (row f of expert e holds column f of the
 *   H x F matrix, i.e. the reduction index h is contiguous); W_down stored
 *   [E,H,F] (row n holds column n of the F x H matrix).
 *
 * Every floating-point step runs in double from the exact input values
 * (bf16 inputs are widened exactly).  Work over tokens / rows is spread over
 * OpenMP threads; each output element is computed by exactly one thread in a
 * fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_EINVAL 1

/* ---------------------------------------------------------------- bf16 --- */

/* Exact widening of a bf16 bit pattern (the top 16 bits of an IEEE binary32). */
double orc_bf16_bits_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * Round a double to the nearest bf16 value (8 significant bits, exponent
 * range of binary32), ties to even.  Done directly from the double, so there
 * is no double rounding through binary32.
 */
double orc_round_to_bf16(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  double m = frexp(x, &e); /* x = m * 2^e, 0.5 <= |m| < 1 */
  /* quantum of the bf16 grid at this binade: 2^(e-8); subnormal floor 2^-133 */
  int q = e - 8;
  if (q < -133) q = -133;
  double scaled = ldexp(x, -q);          /* exact: only changes the exponent */
  double r = nearbyint(scaled);          /* default rounding mode: ties-to-even */
  double y = ldexp(r, q);
  if (fabs(y) >= 0x1p128) y = copysign(INFINITY, x); /* beyond the largest finite bf16 */
  (void)m;
  return y;
}

/* Bits of the bf16 value equal to orc_round_to_bf16(x) (x already on the grid). */
uint16_t orc_double_to_bf16_bits(double x) {
  float f = (float)orc_round_to_bf16(x); /* exact: a bf16 value is a binary32 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* -------------------------------------------------------------- MX fp8 --- */

/*
 * e4m3 ("fn" variant of the OCP 8-bit formats): sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6;
 * the all-ones exponent is a normal binade except code 0x7F/0xFF, NaN.  The
 * largest value is 1.75 * 2^8 = 448.
 */
double orc_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

/* Nearest e4m3 code to v: the non-negative finite codes 0..126 have
 * increasing values, so the two neighbours of |v| are found by bisection
 * and the nearer one taken, a tie going to the even code; magnitudes beyond
 * 448 give 448 (code 126, the largest); the sign bit is v's. */
uint8_t orc_e4m3_round(double v) {
  double a = fabs(v);
  int lo = 0, hi = 126; /* invariant: value(lo) <= a, or lo = 0 */
  if (a >= orc_e4m3_value(126)) {
    lo = 126;
  } else {
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (orc_e4m3_value((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    /* now value(lo) <= a < value(hi), hi = lo + 1 */
    double dl = a - orc_e4m3_value((uint8_t)lo), dh = orc_e4m3_value((uint8_t)hi) - a;
    if (dh < dl || (dh == dl && (hi & 1) == 0)) lo = hi;
  }
  return (uint8_t)(lo | (signbit(v) ? 0x80 : 0));
}

/*
 * MXFP8 block of 32 values (OCP microscaling formats): X = floor(log2 of the
 * largest magnitude) - 8 (8 being the exponent of e4m3's largest value),
 * kept within the scale's range [-127, 127], and -127 for an all-zero block;
 * the scale byte is X + 127; each element is the e4m3 code nearest v / 2^X.
 */
static void mx_block(const double* v, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[i]));
  int X = -127;
  if (amax > 0.0) {
    int e;
    frexp(amax, &e); /* amax = m 2^e, 0.5 <= m < 1: floor(log2 amax) = e - 1 */
    X = e - 1 - 8;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
  }
  for (int i = 0; i < 32; ++i) codes[i] = orc_e4m3_round(ldexp(v[i], -X));
  *scale = (uint8_t)(X + 127);
}

/*
 * Storage of an MX tensor of rows x cols (cols a multiple of 128), the
 * library's buffer format: the codes row by row, then the scale bytes in
 * groups of 32 rows (the last group padded to 32): for row group g and
 * column quad q (columns 128 q .. 128 q + 127, blocks 4 q .. 4 q + 3), 128
 * bytes hold the 4 scale bytes of each of the group's rows, row by row.
 * This is a storage convention only (a kernel reads one stage's scales of
 * 32 rows as 128 contiguous bytes); the values are those of mx_block.
 */
static int64_t mx_scale_index(int64_t r, int b, int cols) {
  return ((r / 32) * (cols / 128) + b / 4) * 128 + (r % 32) * 4 + (b % 4);
}

static int64_t mx_scale_bytes(int64_t rows, int cols) { return (rows + 31) / 32 * 32 * (cols / 32); }

/* Value of element (r, c) of an MX tensor of `cols` columns. */
static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t r, int c, int cols) {
  return ldexp(orc_e4m3_value(codes[r * cols + c]), (int)scales[mx_scale_index(r, c / 32, cols)] - 127);
}

/*
 * Quantise rows x cols values (cols a multiple of 128; f32 or bf16 bits, or
 * doubles when dtype is -1) into one buffer: rows*cols codes, then the
 * scale bytes as above (padding bytes 0).
 */
int orc_mx_quantize(int64_t rows, int cols, int dtype, const void* src, uint8_t* dst) {
  if (rows < 0 || cols < 128 || cols % 128) return ORC_EINVAL;
  uint8_t* scales = dst + rows * (int64_t)cols;
  memset(scales, 0, (size_t)mx_scale_bytes(rows, cols));
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int b = 0; b < cols / 32; ++b) {
      double blk[32];
      for (int i = 0; i < 32; ++i) {
        int64_t idx = r * cols + b * 32 + i;
        blk[i] = dtype < 0 ? ((const double*)src)[idx]
                           : (dtype == ORC_F32 ? (double)((const float*)src)[idx]
                                               : orc_bf16_bits_to_double(((const uint16_t*)src)[idx]));
      }
      mx_block(blk, dst + r * cols + b * 32, scales + mx_scale_index(r, b, cols));
    }
  return ORC_OK;
}

/* Values of a quantised buffer (rows x cols) as doubles. */
int orc_mx_dequantize(int64_t rows, int cols, const uint8_t* src, double* out) {
  if (rows < 0 || cols < 128 || cols % 128) return ORC_EINVAL;
  const uint8_t* scales = src + rows * (int64_t)cols;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) out[r * cols + c] = mx_value(src, scales, r, c, cols);
  return ORC_OK;
}

/* Scale bytes of an MX tensor as a rows x cols/32 array (row-major). */
int orc_mx_scales(int64_t rows, int cols, const uint8_t* src, uint8_t* out) {
  if (rows < 0 || cols < 128 || cols % 128) return ORC_EINVAL;
  const uint8_t* scales = src + rows * (int64_t)cols;
  for (int64_t r = 0; r < rows; ++r)
    for (int b = 0; b < cols / 32; ++b) out[r * (cols / 32) + b] = scales[mx_scale_index(r, b, cols)];
  return ORC_OK;
}

static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  return orc_bf16_bits_to_double(((const uint16_t*)base)[i]);
}

/* --------------------------------------------------------------- route --- */

/*
 * For each token t: the k experts with the largest logits, slot 0 the
 * largest; equal logits go to the lower expert index (IEEE comparison, so
 * -0.0 and +0.0 tie).  Selection k times over the experts not yet taken is
 * the same as taking the first k of the sort by the key (-logit, e).
 * Weights: softmax over the selected logits, shifted by the slot-0 logit.
 */
#define ORC_MAX_EXPERTS 1024 /* size of the per-token selection arrays below */

int orc_route(int64_t M, int E, int k, const float* logits, int32_t* topk_idx, float* topk_w) {
  if (M < 0 || E < 1 || E > ORC_MAX_EXPERTS || k < 1 || k > E) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < M; ++t) {
    const float* row = logits + t * (int64_t)E;
    char taken[ORC_MAX_EXPERTS];
    int sel[ORC_MAX_EXPERTS];
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || row[e] > row[best]) best = e; /* strict: ties keep the lower index */
      }
      taken[best] = 1;
      sel[j] = best;
    }
    double l0 = (double)row[sel[0]];
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += exp((double)row[sel[j]] - l0);
    for (int j = 0; j < k; ++j) {
      topk_idx[t * k + j] = sel[j];
      topk_w[t * k + j] = (float)(exp((double)row[sel[j]] - l0) / denom);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------ segments --- */

/* Number of experts this call holds: EL, or all E when EL is 0. */
static int local_count(int E, int EL) { return EL > 0 ? EL : E; }

static int valid_local(int E, int base, int EL) {
  return base >= 0 && EL >= 0 && (EL == 0 ? base == 0 : base + EL <= E);
}

/* Segment of pair f: src * EL + (expert - base), or -1 if its expert is not
 * held here. */
static int64_t seg_of(const int32_t* topk_idx, const int32_t* src_block, int base, int EL, int k, int64_t f) {
  int64_t t = f / k;
  int64_t s = src_block ? (int64_t)src_block[t] : 0;
  int64_t e = (int64_t)topk_idx[f] - base;
  if (e < 0 || e >= EL) return -1;
  return s * EL + e;
}

/* counts[g] = number of kept pairs in segment g = src*EL + (expert - base);
 * offsets = exclusive prefix sum (offsets[G] = number of kept pairs). */
int orc_counts_offsets(int64_t M, int E, int k, int S, int base, int EL, const int32_t* topk_idx,
                       const int32_t* src_block, int32_t* counts, int32_t* offsets) {
  if (M < 0 || E < 1 || k < 1 || S < 1 || !valid_local(E, base, EL)) return ORC_EINVAL;
  EL = local_count(E, EL);
  int64_t G = (int64_t)S * EL, R = M * k;
  for (int64_t g = 0; g < G; ++g) counts[g] = 0;
  for (int64_t f = 0; f < R; ++f) {
    if (topk_idx[f] < 0 || topk_idx[f] >= E) return ORC_EINVAL;
    int64_t g = seg_of(topk_idx, src_block, base, EL, k, f);
    if (g >= G) return ORC_EINVAL;
    if (g >= 0) counts[g] += 1;
  }
  offsets[0] = 0;
  for (int64_t g = 0; g < G; ++g) offsets[g + 1] = offsets[g] + counts[g];
  return ORC_OK;
}

/* Segment by segment, every kept pair of that segment in increasing flat
 * index; sorted positions past the kept pairs and flat_to_sorted of the
 * dropped pairs hold -1. */
int orc_permutation(int64_t M, int E, int k, int S, int base, int EL, const int32_t* topk_idx,
                    const int32_t* src_block, int32_t* sorted_to_flat, int32_t* flat_to_sorted) {
  if (M < 0 || E < 1 || k < 1 || S < 1 || !valid_local(E, base, EL)) return ORC_EINVAL;
  EL = local_count(E, EL);
  int64_t G = (int64_t)S * EL, R = M * k, r = 0;
  for (int64_t g = 0; g < G; ++g)
    for (int64_t f = 0; f < R; ++f)
      if (seg_of(topk_idx, src_block, base, EL, k, f) == g) sorted_to_flat[r++] = (int32_t)f;
  int64_t kept = r;
  for (; r < R; ++r) sorted_to_flat[r] = -1;
  for (int64_t f = 0; f < R; ++f) flat_to_sorted[f] = -1;
  for (int64_t q = 0; q < kept; ++q) flat_to_sorted[sorted_to_flat[q]] = (int32_t)q;
  return ORC_OK;
}

/* ------------------------------------------------------------ dispatch --- */

/* X_perm[r, :] = x[sorted_to_flat[r] / k, :], a byte copy of the token row;
 * rows whose sorted position holds no pair (-1) are left zero. */
int orc_dispatch(int64_t M, int H, int k, int elem_bytes, const void* x, const int32_t* sorted_to_flat,
                 void* x_perm) {
  if (M < 0 || H < 1 || k < 1 || (elem_bytes != 2 && elem_bytes != 4)) return ORC_EINVAL;
  int64_t R = M * k;
  size_t row = (size_t)H * (size_t)elem_bytes;
  for (int64_t r = 0; r < R; ++r) {
    if (sorted_to_flat[r] < 0) {
      memset((char*)x_perm + (size_t)r * row, 0, row);
      continue;
    }
    int64_t t = sorted_to_flat[r] / k;
    memcpy((char*)x_perm + (size_t)r * row, (const char*)x + (size_t)t * row, row);
  }
  return ORC_OK;
}

/* ----------------------------------------------------------- expert FFN --- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One routed row through expert e: Layer0 (gate and up products, SwiGLU,
 * bf16 rounding of the activation for bf16 layers), then Layer1 (down).
 * xrow is the token row widened to double.  hact [F] and y [H] in double.
 * With act_fp8 the activation is instead quantised to MXFP8 in blocks of 32
 * along F (hact holds the quantised values) and w_down is an MXFP8 buffer
 * of E*H rows of F (codes, then scales).
 */
static void ffn_row(int H, int F, int dtype, int act_fp8, int E, const double* xrow, const void* w_gate,
                    const void* w_up, const void* w_down, int e, double* hact, double* y) {
  int64_t eHF = (int64_t)e * H * F;
  for (int f = 0; f < F; ++f) {
    double g = 0.0, u = 0.0;
    int64_t wrow = eHF + (int64_t)f * H; /* W_gate / W_up stored [E,F,H] */
    for (int h = 0; h < H; ++h) {
      g += xrow[h] * load_elem(w_gate, dtype, wrow + h);
      u += xrow[h] * load_elem(w_up, dtype, wrow + h);
    }
    double a = silu(g) * u;
    /* the quantisation codes are decided on an f32 value, the precision the
       activation has where it is quantised */
    hact[f] = act_fp8 ? (double)(float)a : ((dtype == ORC_BF16) ? orc_round_to_bf16(a) : a);
  }
  if (act_fp8) {
    uint8_t codes[32], sc;
    for (int b = 0; b < F / 32; ++b) {
      mx_block(hact + b * 32, codes, &sc);
      for (int i = 0; i < 32; ++i) hact[b * 32 + i] = ldexp(orc_e4m3_value(codes[i]), (int)sc - 127);
    }
    const uint8_t* wc = (const uint8_t*)w_down;
    const uint8_t* ws = wc + (int64_t)E * H * F;
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      int64_t wrow = (int64_t)e * H + n; /* row of the [E*H, F] tensor */
      for (int f = 0; f < F; ++f) acc += hact[f] * mx_value(wc, ws, wrow, f, F);
      y[n] = acc;
    }
    return;
  }
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    int64_t wrow = eHF + (int64_t)n * F; /* W_down stored [E,H,F] */
    for (int f = 0; f < F; ++f) acc += hact[f] * load_elem(w_down, dtype, wrow + f);
    y[n] = acc;
  }
}

/* Segment g containing sorted row r: offsets[g] <= r < offsets[g+1]. */
static int64_t segment_of_row(const int32_t* offsets, int64_t G, int64_t r) {
  for (int64_t g = 0; g < G; ++g)
    if (offsets[g] <= r && r < offsets[g + 1]) return g;
  return -1;
}

/*
 * Layer0 + Layer1 for a list of sorted rows.  Row r belongs to segment g and
 * uses expert g % E of the weights given (E = the experts held here); its
 * input is X_perm[r] = x[sorted_to_flat[r] / k].
 * hact_out [n_rows, F] and y_out [n_rows, H] in double (either may be NULL).
 */
int orc_ffn_rows(int H, int F, int E, int S, int k, int dtype, int act_fp8, const void* x, const void* w_gate,
                 const void* w_up, const void* w_down, const int32_t* sorted_to_flat, const int32_t* offsets,
                 int64_t n_rows, const int64_t* rows, double* hact_out, double* y_out) {
  if (H < 1 || F < 1 || E < 1 || S < 1 || k < 1 || (dtype != ORC_F32 && dtype != ORC_BF16)) return ORC_EINVAL;
  if (act_fp8 && F % 128) return ORC_EINVAL;
  int64_t G = (int64_t)S * E;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    int64_t g = segment_of_row(offsets, G, r);
    if (g < 0) { bad = 1; continue; }
    int e = (int)(g % E);
    int64_t t = sorted_to_flat[r] / k;
    double* xrow = (double*)malloc(sizeof(double) * (size_t)H);
    double* hact = (double*)malloc(sizeof(double) * (size_t)F);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    for (int h = 0; h < H; ++h) xrow[h] = load_elem(x, dtype, t * H + h);
    ffn_row(H, F, dtype, act_fp8, E, xrow, w_gate, w_up, w_down, e, hact, y);
    if (hact_out) memcpy(hact_out + i * F, hact, sizeof(double) * (size_t)F);
    if (y_out) memcpy(y_out + i * H, y, sizeof(double) * (size_t)H);
    free(xrow); free(hact); free(y);
  }
  return bad ? ORC_EINVAL : ORC_OK;
}

/* -------------------------------------------------------------- combine --- */

/*
 * out[i, :] = sum_{j=0..k-1} w[t,j] * Y[flat_to_sorted[t*k+j], :] for the
 * listed tokens t = tokens[i]; y_rows supplies Y for the pairs of those
 * tokens, in (i, j) order: y_rows[(i*k + j), :] is the row of pair t*k+j.
 * kept (may be NULL: all kept) marks the pairs held here; the others are
 * left out of the sum.
 */
int orc_combine_tokens(int H, int k, int64_t n_tok, const float* topk_w_sub, const double* y_rows,
                       const uint8_t* kept, double* out) {
  if (H < 1 || k < 1) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_tok; ++i) {
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        if (!kept || kept[i * k + j]) acc += (double)topk_w_sub[i * k + j] * y_rows[(i * k + j) * H + n];
      out[i * H + n] = acc;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------- epilogue --- */

/*
 * out[i] = cast(acc[i] + residual[i]) for n values: the residual (NULL: none)
 * widened exactly from res_dtype, the sum in double, then rounded to bf16
 * (round to nearest even) when out_dtype is bf16, else kept.
 */
int orc_epilogue(int64_t n, const double* acc, const void* residual, int res_dtype, int out_dtype, double* out) {
  if (n < 0 || (res_dtype != ORC_F32 && res_dtype != ORC_BF16) || (out_dtype != ORC_F32 && out_dtype != ORC_BF16))
    return ORC_EINVAL;
  for (int64_t i = 0; i < n; ++i) {
    double v = acc[i] + (residual ? load_elem(residual, res_dtype, i) : 0.0);
    out[i] = (out_dtype == ORC_BF16) ? orc_round_to_bf16(v) : v;
  }
  return ORC_OK;
}

/* ---------------------------------------------------------- whole layer --- */

/*
 * The whole layer, in the pages' order: route, segments, permutation over
 * all tokens (always in full), then Layer0/Layer1 and the combine for the
 * listed tokens only (all tokens when tokens == NULL; n_tok must then be M).
 *
 * Outputs: topk_idx/topk_w [M,k], counts [S*E], offsets [S*E+1],
 * sorted_to_flat / flat_to_sorted [M*k] (all full); out [n_tok,H] double;
 * hact [n_tok*k, F] and y [n_tok*k, H] double (may be NULL), row i*k+j
 * belongs to pair (tokens[i], j).
 */
int orc_moe_layer(int64_t M, int H, int F, int E, int k, int S, int base, int EL, int dtype, int act_fp8,
                  const void* x,
                  const float* logits, const int32_t* src_block, const void* w_gate, const void* w_up,
                  const void* w_down, int64_t n_tok, const int64_t* tokens, int32_t* topk_idx, float* topk_w,
                  int32_t* counts, int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted, double* out,
                  double* hact, double* y) {
  int rc = orc_route(M, E, k, logits, topk_idx, topk_w);
  if (rc) return rc;
  rc = orc_counts_offsets(M, E, k, S, base, EL, topk_idx, src_block, counts, offsets);
  if (rc) return rc;
  rc = orc_permutation(M, E, k, S, base, EL, topk_idx, src_block, sorted_to_flat, flat_to_sorted);
  if (rc) return rc;
  if (!tokens && n_tok != M) return ORC_EINVAL;
  EL = local_count(E, EL);

  int64_t n_pairs = n_tok * k;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_pairs > 0 ? n_pairs : 1));
  int64_t* kept_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_pairs > 0 ? n_pairs : 1));
  uint8_t* kept = (uint8_t*)malloc((size_t)(n_pairs > 0 ? n_pairs : 1));
  float* wsub = (float*)malloc(sizeof(float) * (size_t)(n_pairs > 0 ? n_pairs : 1));
  double* yrows = y ? y : (double*)malloc(sizeof(double) * (size_t)(n_pairs > 0 ? n_pairs : 1) * (size_t)H);
  int64_t n_kept = 0;
  for (int64_t i = 0; i < n_tok; ++i) {
    int64_t t = tokens ? tokens[i] : i;
    if (t < 0 || t >= M) { rc = ORC_EINVAL; break; }
    for (int j = 0; j < k; ++j) {
      rows[i * k + j] = flat_to_sorted[t * k + j];
      kept[i * k + j] = rows[i * k + j] >= 0;
      wsub[i * k + j] = topk_w[t * k + j];
      if (kept[i * k + j]) kept_rows[n_kept++] = rows[i * k + j];
    }
  }
  /* the FFN runs for the kept pairs only; a dropped pair's rows hold zeros */
  double* hk = (double*)malloc(sizeof(double) * (size_t)(n_kept > 0 ? n_kept : 1) * (size_t)F);
  double* yk = (double*)malloc(sizeof(double) * (size_t)(n_kept > 0 ? n_kept : 1) * (size_t)H);
  if (!rc)
    rc = orc_ffn_rows(H, F, EL, S, k, dtype, act_fp8, x, w_gate, w_up, w_down, sorted_to_flat, offsets, n_kept,
                      kept_rows, hk, yk);
  if (!rc) {
    int64_t q = 0;
    for (int64_t p = 0; p < n_pairs; ++p) {
      if (kept[p]) {
        memcpy(yrows + p * H, yk + q * H, sizeof(double) * (size_t)H);
        if (hact) memcpy(hact + p * F, hk + q * F, sizeof(double) * (size_t)F);
        ++q;
      } else {
        memset(yrows + p * H, 0, sizeof(double) * (size_t)H);
        if (hact) memset(hact + p * F, 0, sizeof(double) * (size_t)F);
      }
    }
    rc = orc_combine_tokens(H, k, n_tok, wsub, yrows, kept, out);
  }
  free(rows);
  free(kept_rows);
  free(kept);
  free(wsub);
  free(hk);
  free(yk);
  if (!y) free(yrows);
  return rc;
}

/* Number of threads the parallel loops above use (for reporting). */
int orc_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}

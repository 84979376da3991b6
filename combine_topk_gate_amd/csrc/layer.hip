// Fused MoE layer: one persistent kernel, one ordered work queue.
//
// COMET paper review §4.2.1 (thread-block specialisation: data movement and
// GEMM in different thread blocks, the GEMM blocks keep the unfused GEMM
// code) and §4.2.2 (adaptive allocation: the best split depends on the
// shape, is profiled ahead of time and looked up at run time); §4.1.1-§4.1.2
// (Layer0's shared tensor is consumed per M tile; Layer1's per column chunk
// because the Top-K reduction couples a token's rows; the GroupGEMM runs
// column chunk by column chunk so the reduction of the first chunks starts
// early).  PTO MoE article: the seven stages in one kernel, stage hand-offs
// through ready counters with no global barrier, and the number of cores on
// each stage changing while the kernel runs (dynamic AIC grouping).
//
// On one GPU the pages' communication becomes HBM traffic: the gather of
// token rows and the scatter-reduce of expert outputs.  A handful of
// workgroups cannot drive HBM (a copy needs many CUs' worth of loads in
// flight), so the gather is not a stage of this kernel: by default Layer0
// tiles read their token rows straight from x through sorted_to_flat (the
// GEMM loads the rows anyway) and X_perm is not written; with x_perm set,
// the dispatch has copied them and the tiles read X_perm as in the chain.
// What remains is the combine, which runs on workgroups chosen in one of
// two ways:
//   n_mover > 0  workgroups [0, n_mover) are dedicated combiners: they take
//                combine items (column chunk c, block of 32 tokens) in
//                order, each as soon as chunk c's Layer1 tiles are done;
//   n_mover = 0  the combine items sit in the single work queue right after
//                the Layer1 tiles of the next chunk, so whichever
//                workgroup reaches them does them -- the number of
//                workgroups moving data grows when the matrix work runs out.
// The queue: every Layer0 tile; then per column chunk c its Layer1 tiles
// (each waits until all Layer0 column tiles of its M-tile are done),
// followed (dynamic mode) by the combine items of chunk c-1; finally the
// combine items of the last chunk.  Items are claimed with an atomic
// counter in queue order and every wait targets items earlier in that
// order, held by resident workgroups, so the kernel cannot deadlock when
// the whole grid is resident (one workgroup per CU).  Counters in the
// workspace are the flags: l0done[mt] (Layer0 column tiles of M-tile mt
// finished) and chunkdone[c] (Layer1 tiles of chunk c finished).
// Producers publish with an agent-scope release; consumers spin (bounded)
// and acquire.  A wait that exceeds its bound records a timeout in the
// status word; every workgroup then stops.
//
// Results are bit-identical to the kernel chain: the tiles run the same
// tile routine on the same values in the same k order, and the combine
// uses the same per-element routine.
#include <cstdlib>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "common.hpp"
#include "gemm_bf16.hpp"
#include "launch.hpp"
#include "layer.hpp"
#include "tiles.hpp"

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

constexpr int kChunkTiles = 4;      // Layer1 column tiles per combine chunk (4 x 256 columns)
constexpr int kCombineTokens = 32;  // tokens per combine work item
constexpr int kDefaultSpin = 1 << 22;

struct FusedGeom {
  int mt_max;  // upper bound of M-tiles
  int nc;      // combine chunks
};

static FusedGeom fused_geom(int64_t M, int H, int k, int G) {
  FusedGeom f;
  const int64_t R = M * k;
  f.mt_max = (int)((R + kTileRows - 1) / kTileRows) + G;
  const int nt1 = (H + kL1Cols - 1) / kL1Cols;
  f.nc = (nt1 + kChunkTiles - 1) / kChunkTiles;
  return f;
}

// flags: l0done[mt_max], chunkdone[nc], queue counters [kXcds + 1]
constexpr int kQueueWords = kXcds + 1;

size_t fused_ws_bytes(int64_t M, int H, int F, int E, int k, int S) {
  (void)F;
  const FusedGeom f = fused_geom(M, H, k, S * E);
  return (size_t)(f.mt_max + f.nc + kQueueWords) * sizeof(int32_t);
}

// ---------------------------------------------------------------- flags ---
__device__ __forceinline__ int ld_flag(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 spins until *flag >= target (bounded); the block learns the
// outcome through LDS.  false: timed out here or elsewhere (status set).
__device__ bool block_wait(const int32_t* flag, int target, int32_t* status, int limit, int* lds_word) {
  if (threadIdx.x == 0) {
    int ok = 1;
    int polls = 0;
    while (ld_flag(flag) < target) {
      if (ld_flag(status) != kStatusOk) {
        ok = 0;
        break;
      }
      if (++polls > limit) {
        __hip_atomic_store(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *lds_word = ok;
  }
  __syncthreads();
  const bool ok = *lds_word != 0;
  __syncthreads();
  return ok;
}

// The block's global writes, then one agent-scope release add by thread 0
// (the workgroup barrier orders the other waves' writes before it).
__device__ void block_signal(int32_t* flag, int add) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(flag, add, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Next item of a queue counter, shared with the whole block.
__device__ int block_claim(int32_t* counter, int* lds_word) {
  if (threadIdx.x == 0) *lds_word = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int v = *lds_word;
  __syncthreads();
  return v;
}

// out[t, columns of chunk c] for tokens [t0, t1) (t1 - t0 <= kCombineTokens).
// The tokens' held slots (row index and weight, in slot order; a row outside
// [0, M k) is a pair of an expert not held here) are compacted in LDS, with
// their count per token.  Each thread then owns one 4-column group and walks
// the tokens 16 at a time, two held slots per step: the 32 row loads of a
// step are all issued before any is used, and a group takes as many steps
// as its tokens' largest count needs (one load at a time per thread left a
// combine item ~4x slower than the memory allows).  Per element the
// arithmetic is combine_group's: from zero, held slots in order, one fmaf
// each.
__device__ void combine_chunk(const FusedArgs& a, int c, int64_t t0, int64_t t1, int* rows_lds, float* w_lds,
                              int* cnt_lds) {
  const int n0 = c * kChunkTiles * kL1Cols;
  const int n1 = min(a.H, n0 + kChunkTiles * kL1Cols);
  const int groups = (n1 - n0) / 4;
  const int nt = (int)(t1 - t0), k = a.k;
  const uint64_t R = (uint64_t)(a.M * k);
  for (int i = threadIdx.x; i < nt * k; i += kGemmThreads) {
    rows_lds[i] = a.f2s[t0 * k + i];
    w_lds[i] = a.topk_w[t0 * k + i];
  }
  __syncthreads();
  if (threadIdx.x < nt) {  // in place: the write index never passes the read index
    const int i = threadIdx.x;
    int n = 0;
    for (int j = 0; j < k; ++j) {
      const int32_t row = rows_lds[i * k + j];
      if ((uint64_t)(int64_t)row >= R) continue;
      rows_lds[i * k + n] = row;
      w_lds[i * k + n] = w_lds[i * k + j];
      ++n;
    }
    cnt_lds[i] = n;
  }
  __syncthreads();
  constexpr int U = 16;
  for (int q = threadIdx.x; q < groups; q += kGemmThreads) {
    const int64_t n = n0 + 4 * q;
    for (int i0 = 0; i0 < nt; i0 += U) {
      int hmax = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) hmax = max(hmax, cnt_lds[min(i0 + u, nt - 1)]);
      hmax = uniform(hmax);  // the same LDS values in every lane
      float4 acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int h0 = 0; h0 < hmax; h0 += 2) {
        float4 v[2][U];
        float wv[2][U];
        bool has[2][U];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int i = min(i0 + u, nt - 1);
            has[h][u] = h0 + h < cnt_lds[i];
            const int32_t row = has[h][u] ? rows_lds[i * k + h0 + h] : 0;
            wv[h][u] = has[h][u] ? w_lds[i * k + h0 + h] : 0.f;
            v[h][u] = has[h][u] ? *reinterpret_cast<const float4*>(a.y + (int64_t)row * a.H + n)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (!has[h][u]) continue;
            acc[u].x = fmaf(wv[h][u], v[h][u].x, acc[u].x);
            acc[u].y = fmaf(wv[h][u], v[h][u].y, acc[u].y);
            acc[u].z = fmaf(wv[h][u], v[h][u].z, acc[u].z);
            acc[u].w = fmaf(wv[h][u], v[h][u].w, acc[u].w);
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u < nt) store_out(a.out, (t0 + i0 + u) * a.H + n, acc[u]);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kGemmThreads) void fused_layer_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLdsBytes];
  __shared__ TileLds tl;
  __shared__ int lds_word;
  __shared__ int comb_rows[kCombineTokens * 16];
  __shared__ float comb_w[kCombineTokens * 16];
  __shared__ int comb_cnt[kCombineTokens];

  const int MT = build_tile_table(a.offsets, a.G, kTileRows, tl);
  const int nt0 = (a.F + kL0Cols - 1) / kL0Cols;
  const int nt1 = (a.H + kL1Cols - 1) / kL1Cols;
  const int nc = (nt1 + kChunkTiles - 1) / kChunkTiles;
  int32_t* l0done = a.flags;
  int32_t* chunkdone = a.flags + a.mt_max;
  int32_t* mover_q = chunkdone + nc;
  int32_t* xcd_q = mover_q + 1;
  const int limit = a.spin_limit > 0 ? a.spin_limit : kDefaultSpin;
  const int CB = (int)((a.M + kCombineTokens - 1) / kCombineTokens);  // combine items per chunk
  const bool dedicated = a.n_mover > 0;
  auto chunk_width = [&](int c) { return min(kChunkTiles, nt1 - c * kChunkTiles); };
  auto chunk_items = [&](int c) { return MT * chunk_width(c); };  // queue entries of chunk c's Layer1 tiles
  // reordering check: items permuted inside their section (Layer0 tiles,
  // one chunk's Layer1 tiles, one chunk's combine items); waits still
  // target earlier sections only
  const Shuffle s_cb = make_shuffle(a.shuffle, CB);

  if ((int)blockIdx.x < a.n_mover) {
    // dedicated combiners: chunk by chunk, token blocks in order
    for (;;) {
      const int v = block_claim(mover_q, &lds_word);
      if (v >= nc * CB) return;
      const int c = v / CB, tb = shuffled(s_cb, v - c * CB);
      if (!block_wait(chunkdone + c, chunk_items(c), a.status, limit, &lds_word)) return;
      combine_chunk(a, c, (int64_t)tb * kCombineTokens, min(a.M, (int64_t)(tb + 1) * kCombineTokens), comb_rows,
                    comb_w, comb_cnt);
    }
  }

  // the single ordered queue of the other workgroups
  const int T0 = MT * nt0;
  int total = T0;
  for (int c = 0; c < nc; ++c) total += chunk_items(c) + ((dedicated || c == 0) ? 0 : CB);
  if (!dedicated) total += CB;
  const int W = gridDim.x - a.n_mover;
  const int xcd_slots = W / kXcds > 0 ? W / kXcds : 1;
  // The queue is dealt to the XCDs in runs of `run` items (run r to queue
  // r % nq), and the workgroups of one XCD (hardware ids b with the same
  // b % 8) claim from their queue's counter: the tiles running at once on
  // an XCD are neighbours in the order and share its L2.  Claims stay in
  // increasing order per queue, which keeps the no-deadlock argument.
  const int nq = ((W % kXcds) == 0 && (a.n_mover % kXcds) == 0) ? kXcds : 1;
  const int run = xcd_slots;
  const int q = (nq == 1) ? 0 : (int)(blockIdx.x % kXcds);
  int32_t* my_q = xcd_q + q;
  const Shuffle s_l0 = make_shuffle(a.shuffle, T0);
  Bf16GemmArgs ga;
  ga.E = a.E;
  ga.s2f = a.s2f;
  ga.topk = a.k;
  ga.M = a.M;
  for (;;) {
    const int i = block_claim(my_q, &lds_word);
    const int v = (i / run) * (nq * run) + q * run + (i % run);
    if (v >= total) return;
    if (v < T0) {
      const TileCoord c = tile_coord(shuffled(s_l0, v), a.G, nt0, kTileRows, xcd_slots, (int64_t)kTileRows * a.H * 2, tl);
      ga.w0 = reinterpret_cast<const __bf16*>(a.w_gate);
      ga.w1 = reinterpret_cast<const __bf16*>(a.w_up);
      ga.c = a.hact;
      ga.K = a.H;
      ga.N = a.F;
      if (a.x_perm) {
        ga.a = reinterpret_cast<const __bf16*>(a.x_perm);
        bf16_gemm_row_tile<0>(ga, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
      } else {
        ga.a = reinterpret_cast<const __bf16*>(a.x);
        bf16_gemm_row_tile<0, true>(ga, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, c.nt, lds);
      }
      block_signal(l0done + c.mt, 1);
      continue;
    }
    // locate v among the chunk sections
    int u = v - T0, chunk = 0;
    bool is_tile = false;
    int comb_chunk = -1;
    for (; chunk <= nc; ++chunk) {
      if (chunk < nc) {
        const int n = chunk_items(chunk);
        if (u < n) {
          is_tile = true;
          break;
        }
        u -= n;
      }
      if (!dedicated && chunk >= 1) {
        if (u < CB) {
          comb_chunk = chunk - 1;
          break;
        }
        u -= CB;
      }
    }
    if (is_tile) {
      const int ui = shuffled(make_shuffle(a.shuffle, chunk_items(chunk)), u);
      const TileCoord c = tile_coord(ui, a.G, chunk_width(chunk), kTileRows, xcd_slots, (int64_t)kTileRows * a.F * 2, tl);
      if (!block_wait(l0done + c.mt, nt0, a.status, limit, &lds_word)) return;
      ga.a = reinterpret_cast<const __bf16*>(a.hact);
      ga.w0 = reinterpret_cast<const __bf16*>(a.w_down);
      ga.w1 = nullptr;
      ga.c = a.y;
      ga.K = a.F;
      ga.N = a.H;
      bf16_gemm_row_tile<1>(ga, c.g, tl.seg_start[c.g], tl.seg_rows[c.g], c.m0, chunk * kChunkTiles + c.nt, lds);
      block_signal(chunkdone + chunk, 1);
    } else if (comb_chunk >= 0) {
      if (!block_wait(chunkdone + comb_chunk, chunk_items(comb_chunk), a.status, limit, &lds_word)) return;
      const int tb = shuffled(s_cb, u);
      combine_chunk(a, comb_chunk, (int64_t)tb * kCombineTokens, min(a.M, (int64_t)(tb + 1) * kCombineTokens),
                    comb_rows, comb_w, comb_cnt);
    }
  }
}

// -------------------------------------------------------- split table ---
// Per-shape plan, profiled on MI355X (256 CUs, one workgroup per CU) with
// combine_topk_gate_amd/tune_split.py: the number of dedicated combine
// workgroups of the fused kernel (0: combine items in the shared queue), or
// -1 where the kernel chain was faster than every fused split.  Shapes not
// listed run the chain too: on one MI355X the chain was faster on every
// shape measured, from 300 tokens (47 vs 76 us) to the listed layers, so
// the fused kernel runs where a caller asks for it (opts->n_mover >= 0).
// COMET paper review §4.2.2: the split is profiled ahead of time, stored as
// metadata and looked up at run time.  The table below is the one stored in
// combine_topk_gate_amd/tuning/mi355x.json; MOE_TUNING_TABLE=<path> makes
// the library use the entries of that JSON file instead (written by
// tune_split.py --write on the target GPU).
struct SplitEntry {
  int64_t M;
  int H, F, E, k, S, EL, movers;  // EL: experts held (E when all are)
};
static const SplitEntry kSplitTable[] = {
    {4096, 2048, 1408, 64, 4, 1, 64, -1},
    {8192, 4096, 14336, 8, 2, 1, 8, -1},
    {16384, 4096, 6400, 16, 2, 1, 16, -1},
    {16384, 7168, 4096, 16, 8, 8, 16, -1},
    {16384, 7168, 4096, 128, 8, 8, 16, -1},  // 16 of 128 experts held
};

namespace {

// A small reader for the table file: {"entries": [{"M": 8192, "H": 4096,
// "F": 14336, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": -1, ...}, ...]}.
// Every entry needs those eight integer keys; other keys (strings, numbers,
// true/false/null) are skipped, and so is everything outside "entries".
struct TableReader {
  const std::string& t;
  size_t i = 0;
  explicit TableReader(const std::string& text) : t(text) {}
  void ws() {
    while (i < t.size() && (t[i] == ' ' || t[i] == '\n' || t[i] == '\r' || t[i] == '\t')) ++i;
  }
  bool eat(char c) {
    ws();
    if (i < t.size() && t[i] == c) {
      ++i;
      return true;
    }
    return false;
  }
  bool string(std::string* out) {
    if (!eat('"')) return false;
    std::string s;
    while (i < t.size() && t[i] != '"') {
      if (t[i] == '\\') {
        if (++i >= t.size()) return false;
      }
      s += t[i++];
    }
    if (i >= t.size()) return false;
    ++i;
    if (out) *out = s;
    return true;
  }
  // a JSON number; *integral tells whether it has no fraction or exponent
  bool number(double* v, bool* integral) {
    ws();
    const size_t j = i;
    if (i < t.size() && t[i] == '-') ++i;
    bool digits = false, frac = false;
    while (i < t.size() && ((t[i] >= '0' && t[i] <= '9') || t[i] == '.' || t[i] == 'e' || t[i] == 'E' ||
                            ((t[i] == '+' || t[i] == '-') && i > j && (t[i - 1] == 'e' || t[i - 1] == 'E')))) {
      if (t[i] >= '0' && t[i] <= '9') digits = true; else frac = true;
      ++i;
    }
    if (!digits) return false;
    char* end = nullptr;
    const std::string s = t.substr(j, i - j);
    *v = std::strtod(s.c_str(), &end);
    *integral = !frac;
    return end && *end == 0;
  }
  bool literal() {
    ws();
    for (const char* w : {"true", "false", "null"}) {
      const size_t n = std::char_traits<char>::length(w);
      if (t.compare(i, n, w) == 0) {
        i += n;
        return true;
      }
    }
    return false;
  }
  // skips any value (for keys outside "entries")
  bool skip_value() {
    ws();
    if (i >= t.size()) return false;
    if (t[i] == '"') return string(nullptr);
    if (t[i] == '{' || t[i] == '[') {
      const char close = t[i] == '{' ? '}' : ']';
      const bool obj = t[i] == '{';
      ++i;
      if (eat(close)) return true;
      do {
        if (obj && (!string(nullptr) || !eat(':'))) return false;
        if (!skip_value()) return false;
      } while (eat(','));
      return eat(close);
    }
    if (literal()) return true;
    double v;
    bool integral;
    return number(&v, &integral);
  }
  bool entry(SplitEntry* e) {
    if (!eat('{')) return false;
    static const char* keys[8] = {"M", "H", "F", "E", "k", "S", "EL", "n_mover"};
    int64_t val[8];
    bool seen[8] = {false, false, false, false, false, false, false, false};
    if (!eat('}')) {
      do {
        std::string key;
        if (!string(&key) || !eat(':')) return false;
        int which = -1;
        for (int q = 0; q < 8; ++q)
          if (key == keys[q]) which = q;
        if (which < 0) {
          if (!skip_value()) return false;
          continue;
        }
        double v;
        bool integral;
        if (!number(&v, &integral) || !integral || v < -1 || v > 9.0e15) return false;
        val[which] = (int64_t)v;
        seen[which] = true;
      } while (eat(','));
      if (!eat('}')) return false;
    }
    for (int q = 0; q < 8; ++q)
      if (!seen[q]) return false;
    for (int q = 1; q < 8; ++q)
      if (val[q] > 0x7fffffff) return false;
    *e = SplitEntry{val[0], (int)val[1], (int)val[2], (int)val[3], (int)val[4], (int)val[5], (int)val[6], (int)val[7]};
    return true;
  }
  bool table(std::vector<SplitEntry>* out) {
    if (!eat('{')) return false;
    bool found = false;
    if (!eat('}')) {
      do {
        std::string key;
        if (!string(&key) || !eat(':')) return false;
        if (key != "entries") {
          if (!skip_value()) return false;
          continue;
        }
        if (found || !eat('[')) return false;
        found = true;
        if (!eat(']')) {
          do {
            SplitEntry e;
            if (!entry(&e)) return false;
            out->push_back(e);
          } while (eat(','));
          if (!eat(']')) return false;
        }
      } while (eat(','));
      if (!eat('}')) return false;
    }
    ws();
    return found && i == t.size();
  }
};

std::mutex g_table_mu;
std::string g_table_path;           // file the entries below came from
std::vector<SplitEntry> g_table;    // its entries
bool g_table_ok = false;

// The plan of a shape from the entries in use: the file MOE_TUNING_TABLE
// names (read when the variable first takes that value), else the
// compiled-in table.  kTableUnusable: the variable is set but the file
// cannot be read or parsed.  No allocation once the file has been read.
int table_lookup(int64_t M, int H, int F, int E, int k, int S, int EL, int cus) {
  auto find = [&](const SplitEntry* b, const SplitEntry* e) {
    for (const SplitEntry* s = b; s != e; ++s)
      if (s->M == M && s->H == H && s->F == F && s->E == E && s->k == k && s->S == S && s->EL == EL)
        return s->movers < 0 ? -1 : (s->movers < cus ? s->movers : 0);
    return -1;
  };
  const char* path = std::getenv("MOE_TUNING_TABLE");
  if (!path || !*path) return find(std::begin(kSplitTable), std::end(kSplitTable));
  std::lock_guard<std::mutex> lock(g_table_mu);
  if (g_table_path != path) {
    g_table_path = path;
    g_table.clear();
    std::ifstream f(path, std::ios::binary);
    std::stringstream buf;
    if (f) buf << f.rdbuf();
    const std::string text = buf.str();
    TableReader r(text);
    g_table_ok = f.good() || f.eof() ? r.table(&g_table) : false;
    if (!g_table_ok) g_table.clear();
  }
  if (!g_table_ok) return kTableUnusable;
  return find(g_table.data(), g_table.data() + g_table.size());
}

}  // namespace

int fused_default_movers(int64_t M, int H, int F, int E, int k, int S, int EL, int dtype, int cus) {
  if (dtype != MOE_DTYPE_BF16) return -1;
  return table_lookup(M, H, F, E, k, S, EL, cus);
}

int fused_mt_max(int64_t M, int H, int k, int G) { return fused_geom(M, H, k, G).mt_max; }

// Workgroups of the fused kernel one CU holds at once (LDS and registers).
static int fused_blocks_per_cu() {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_layer_kernel, kGemmThreads, 0) != hipSuccess) n = 0;
    cached = n;
  }
  return cached;
}

moe_status_t fused_check(const FusedArgs& a, int cus) {
  // every workgroup must be resident at once, or a wait could target work
  // that has not been scheduled
  if (a.grid < 1 || a.grid > cus * fused_blocks_per_cu()) return MOE_ERR_UNSUPPORTED;
  if (a.n_mover < 0 || a.n_mover >= a.grid) return MOE_ERR_INVALID_ARGUMENT;
  const FusedGeom f = fused_geom(a.M, a.H, a.k, a.G);
  if (a.mt_max != f.mt_max) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

int fused_flag_words(int64_t M, int H, int k, int G) {
  const FusedGeom f = fused_geom(M, H, k, G);
  return f.mt_max + f.nc + kQueueWords;
}

// a.flags (fused_flag_words of them) must be zero: cleared on the stream
// before this launch
hipError_t launch_fused_layer(const FusedArgs& a, hipStream_t s) {
  fused_layer_kernel<<<a.grid, kGemmThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe

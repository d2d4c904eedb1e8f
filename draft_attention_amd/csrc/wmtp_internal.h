// wmtp_internal.h -- declarations shared by the translation units of libwmtp.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "wmtp.h"

namespace wmtp {

// Work split of one attention call (split-K flash decoding). The keys of every (sequence, KV head,
// row chunk) are dealt in 16-key tiles over n_splits workgroups; each workgroup leaves one
// un-normalised partial result (o, running max, running sum) in the workspace, which a second
// kernel merges with the log-sum-exp rule. The plan depends only on the call's sizes.
struct SplitPlan {
  int G;               // query heads per KV head
  int rows;            // G * m query rows per KV head
  int n_chunks;        // row chunks handled by separate wavefronts
  int chunk_rows;      // rows of a chunk (the last one may hold fewer)
  bool coop;           // cooperative-tile kernel (else the key-split kernel)
  int nr;              // 16-row MFMA blocks per chunk
  int n_splits;        // workgroups (partials) per (sequence, KV head, chunk)
  bool q_lds;          // key-split kernel: query operand loaded once per workgroup into LDS
  size_t ws_o_floats;  // partial outputs: [bhc][n_splits][16*nr][head_dim]
  size_t ws_ml_floats; // running max and sum: [bhc][n_splits][16*nr][2]
};

constexpr int kTileKeys = 16;       // keys per MFMA tile
constexpr int kWavesPerBlock = 4;   // wavefronts per workgroup (interleaved tiles of one range)
// Build-time tuning knobs (hipcc -D...), each defaulting to the value measured best on MI355X:
//   WMTP_TARGET_BLOCKS_SPLIT / _COOP  workgroups per call of each attention kernel (below)
//   WMTP_ALLOW_COOP                   0: every row count on the key-split kernel
//   WMTP_COOP_TPS, WMTP_COOP_PREFETCH tiles per LDS stage, stages in flight (cooperative kernel)
//   WMTP_COOP_WPC                     workgroups per CU the cooperative kernel is compiled for
//   WMTP_COOP_EIGHT_WAVES             0: eight row blocks on four wavefronts (two blocks each)
//   WMTP_MIN_TILES_PER_WAVE           smallest share of a wavefront when the planner splits keys
// workgroups per call (256 CUs), measured best for each kernel on MI355X at L = 1M
#ifndef WMTP_TARGET_BLOCKS_SPLIT
#define WMTP_TARGET_BLOCKS_SPLIT 256
#endif
#ifndef WMTP_TARGET_BLOCKS_COOP
#define WMTP_TARGET_BLOCKS_COOP 512
#endif
#ifndef WMTP_ALLOW_COOP
#define WMTP_ALLOW_COOP 1
#endif
constexpr int kTargetBlocksSplit = WMTP_TARGET_BLOCKS_SPLIT;
constexpr int kTargetBlocksCoop = WMTP_TARGET_BLOCKS_COOP;
constexpr bool kAllowCoop = WMTP_ALLOW_COOP != 0;
constexpr int kMaxCapacity = 1 << 30;  // keeps key indices below 2^31
constexpr int kMaxM = 16;           // verify candidates per call

// Plan for a cache of `dtype`; false when no attention call accepts these sizes.
bool make_plan_for(int batch, int n_q_heads, int n_kv_heads, int head_dim, int m,
                   int max_seq_len, int dtype, SplitPlan* plan);

enum AttnMode { kModeWindowed = 0, kModeFull = 1, kModeVerify = 2 };

// Division by a value fixed for a whole call (head counts, group size, candidates, row chunks) as
// one multiply-high, an add and a shift, exact for dividends below 2^31 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI 1994, the round-up
// multiplier): with s = ceil(log2 d) and mul = floor(2^32 (2^s - d) / d) + 1,
// x / d = (umulhi(x, mul) + x) >> s. A run-time division otherwise costs a dependent sequence of
// about twenty instructions, several of which stand between a kernel's start and its first load.
struct FastDiv {
  uint32_t d, mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d < 1 ? 1 : d;
  f.shift = 0;
  while ((1ull << f.shift) < f.d) ++f.shift;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << f.shift) - f.d)) / f.d + 1);
  return f;
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_len;
  float* out;
  float* lse;
  float* ws_o;
  float* ws_ml;
  int batch, n_kv_heads, n_q_heads, head_dim, m, capacity;
  int limit;  // keys beyond min(seq_len, limit) are never read
  int mode;
  float sm_scale;
  // windowed mode on a ring with slack (wphys > window): key i of the attended set lives in slot
  // i for the min(S, n) sinks, else in slot S + (w0 - S + i - sinks) mod wphys with
  // w0 = max(sinks, n - window). With wphys == window the attended keys are slots 0..limit-1.
  int sink, window, wphys;
  // partial results of split s of (sequence, KV head, chunk) bhc go to index
  // bhc * part_stride + part_offset + s (two launches can fill one merge: MASW working memory)
  int part_stride, part_offset;
  // fused draft step (split kernel, one row block): append one token per sequence, then attend.
  // new_k/new_v [batch][1][n_kv_heads][head_dim] (NULL otherwise). The split kernel reads the new
  // token from there, workgroup (split 0, chunk 0) of each KV head copies it into its slot (and
  // pos), and the merge kernel advances seq_len afterwards (no attention workgroup sees the bump).
  const void* new_k;
  const void* new_v;
  int32_t* pos;
  // divisors of the index arithmetic, filled by the launchers from the sizes above and the plan:
  // n_q_heads, n_kv_heads, G = n_q_heads / n_kv_heads, m, row chunks, rows per chunk
  FastDiv div_hq, div_kv, div_g, div_m, div_chunks, div_crows;
};

// split kernel (or cooperative kernel) writing partials, then the log-sum-exp merge over
// part_stride partials per (sequence, KV head, chunk)
hipError_t launch_attention(const AttnArgs& a, const SplitPlan& p, int dtype, hipStream_t stream);
hipError_t launch_partials(const AttnArgs& a, const SplitPlan& p, int dtype, hipStream_t stream);
hipError_t launch_merge(const AttnArgs& a, const SplitPlan& p, int total_splits, hipStream_t stream);

struct AppendArgs {
  void* k;
  void* v;
  int32_t* pos;
  int32_t* seq_len;
  const void* k_new;
  const void* v_new;
  int batch, n_kv_heads, head_dim, capacity, sink, window, n_new, elem_bytes;
};

// `window` is the physical window of a ring (capacity - sink; 0 for a contiguous cache).
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

struct RollbackArgs {
  int32_t* pos;
  int32_t* seq_len;
  const int32_t* n_drop;
  int batch, capacity, sink;
  int window;  // physical window (capacity - sink) of a ring, 0 for a contiguous cache
  int slack;   // ring: tokens that can be discarded exactly (capacity - sink - attended window)
};

hipError_t launch_rollback(const RollbackArgs& a, hipStream_t stream);

struct AcceptArgs {
  const void* logits;  // [batch][k+1][vocab]
  const int32_t* draft;  // [batch][k]
  int32_t* choice;       // [batch][k+1]
  int32_t* n_accept;     // [batch]
  int32_t* next_token;   // [batch]
  int32_t* n_drop;       // [batch]
  float* ws_val;         // [batch*(k+1)][chunks]
  int32_t* ws_idx;       // [batch*(k+1)][chunks]
  int batch, k, vocab, chunks, dtype;
};

constexpr int kAcceptChunk = 4096;  // vocabulary entries per argmax workgroup
hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);

}  // namespace wmtp

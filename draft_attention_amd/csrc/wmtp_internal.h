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
  size_t ws_o_floats;  // partial outputs: [bhc][n_splits][16*nr][head_dim]
  size_t ws_ml_floats; // running max and sum: [bhc][n_splits][16*nr][2]
};

constexpr int kTileKeys = 16;       // keys per MFMA tile
constexpr int kWavesPerBlock = 4;   // wavefronts per workgroup (interleaved tiles of one range)
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
};

hipError_t launch_attention(const AttnArgs& a, const SplitPlan& p, int dtype, hipStream_t stream);

struct AppendArgs {
  void* k;
  void* v;
  int32_t* pos;
  int32_t* seq_len;
  const void* k_new;
  const void* v_new;
  int batch, n_kv_heads, head_dim, capacity, sink, window, n_new, elem_bytes;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

}  // namespace wmtp

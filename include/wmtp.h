/*
 * wmtp.h -- C ABI of libwmtp.so: Windowed-MTP draft attention, the full-context draft attention it
 * replaces, and the target's full-attention verification, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Windowed-MTP abstract (thelatestinai.com/papers/2607.21535; the same
 * text is on the khansong-paper-with-me page):
 *   - a native MTP draft head runs full attention over the entire KV cache at every draft step
 *     (third sentence)                                      -> wmtp_draft_attn_full
 *   - the draft may take several steps, each of which appends its token first (fourth sentence)
 *                                                            -> wmtp_ring_append + an attention call
 *   - Windowed-MTP gives only the draft's attention a StreamingLLM-style set of attention sinks plus
 *     a sliding window, leaving full-attention verification intact (fifth sentence)
 *                                                            -> wmtp_draft_attn_windowed,
 *                                                               wmtp_verify_attn
 *   - the draft KV that is never read is reclaimed by a compact ring buffer (last sentence)
 *                                                            -> the ring layout of wmtp_kv
 * and the steps around them in a speculative iteration:
 *   - a draft step appends its token and attends            -> wmtp_draft_step_windowed/_full
 *   - the target appends the candidates and verifies them   -> wmtp_verify_step
 *   - greedy accept/reject, then discarding rejected speculative KV (MASW page, sections 1 and
 *     4.3)                                                   -> wmtp_greedy_accept, wmtp_ring_rollback
 *   - the MASW working memory of sinks, memory slots and a local window (MASW page, section 4.1)
 *                                                            -> wmtp_draft_attn_masw
 *
 * Conventions (the pages fix none of them; these are the library's):
 *   - Positions: the tokens of sequence b are numbered 0, 1, 2, ... in append order; seq_len[b] is
 *     how many have been appended. Attention sinks are positions 0..sink-1; the window is the last
 *     `window` positions, the newest included; a position in both sets is attended once.
 *   - Slot map: position p lives in slot p if p < sink, else in slot
 *     sink + (p - sink) % (capacity - sink) (= % window for a ring without slack slots).
 *     A contiguous (non-ring) cache is the same descriptor with window = 0 and sink = capacity, so
 *     that slot(p) = p.
 *   - GQA: query head hq reads KV head hq / G, G = n_q_heads / n_kv_heads (contiguous groups).
 *   - Layouts are dense, row-major, C order:
 *       cache K and V      [batch][n_kv_heads][capacity][head_dim]   (dtype of the cache)
 *       pos                [batch][capacity] int32                    (optional)
 *       seq_len            [batch] int32
 *       new tokens         [batch][n_new][n_kv_heads][head_dim]       (dtype of the cache)
 *       q                  [batch][m][n_q_heads][head_dim]            (dtype of the cache; m = 1
 *                                                                      for a draft step)
 *       out                [batch][m][n_q_heads][head_dim] float32
 *       lse                [batch][m][n_q_heads] float32, natural log (optional)
 *   - Scores are sm_scale * (q . k); softmax and all accumulation are float32. bf16 operands are
 *     multiplied exactly; the softmax weights are rounded to bf16 for the weighted sum of V.
 *
 * Ownership and execution: every pointer inside wmtp_kv and every q/out/lse/ws/k_new/v_new pointer
 * is DEVICE memory owned by the caller. The library never allocates, frees or synchronises; it
 * keeps no global state, so calls from several host threads are safe. Every call only enqueues work
 * on `stream` (a hipStream_t; NULL = the null stream) and returns; buffers must stay alive and
 * unmodified until the stream has passed the call. The wmtp_kv descriptor itself is host memory and
 * is read only during the call.
 *
 * Errors: every entry point validates its host-side arguments first and returns a nonzero
 * wmtp_status WITHOUT launching anything or touching any buffer when they are invalid. A HIP launch
 * failure returns WMTP_ERR_HIP. No C++ exception or abort crosses this ABI. Device-side contents
 * (seq_len, the data) cannot be validated on the host; the kernels never access memory outside the
 * buffers described, whatever seq_len holds (see each call). Rows (ring slots) at or past a
 * sequence's length may hold any bytes, NaN and Inf included: the attention calls may read them
 * but they never reach out or lse, so a cache need not be cleared when it is allocated.
 */
#ifndef WMTP_H
#define WMTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wmtp_status {
  WMTP_OK = 0,
  WMTP_ERR_INVALID_ARG = 1, /* null pointer, inconsistent sizes, bad descriptor */
  WMTP_ERR_UNSUPPORTED = 2, /* dtype, head_dim or group shape the kernels do not implement */
  WMTP_ERR_CAPACITY = 3,    /* a request that cannot fit (n_new larger than a contiguous cache) */
  WMTP_ERR_WORKSPACE = 4,   /* workspace missing or smaller than wmtp_attn_workspace_bytes */
  WMTP_ERR_HIP = 5          /* the HIP runtime reported an error at launch */
} wmtp_status;

typedef enum wmtp_dtype { WMTP_F32 = 0, WMTP_BF16 = 1 } wmtp_dtype;

/* A KV cache of `batch` sequences: a compact ring buffer (window >= 1, capacity >= sink + window) or
 * a contiguous cache (window = 0, sink = capacity). head_dim must be 64, 128 or 256;
 * 1 <= capacity <= 2^30 (larger capacities return WMTP_ERR_CAPACITY); 1 <= batch <= 65535, and an
 * attention call needs batch * n_kv_heads * (row chunks per KV head) <= 65535, a row chunk holding
 * 16 to 128 of a KV head's query rows (m * n_q_heads / n_kv_heads) depending on dtype and head_dim
 * (INVALID_ARG otherwise).
 * A ring's window positions wrap over its capacity - sink window slots: slot(p) = p for p < sink,
 * else sink + (p - sink) % (capacity - sink). The draft attends the sinks and the last `window`
 * positions; the slack = capacity - sink - window extra slots let up to `slack` of the newest
 * tokens be discarded again exactly (wmtp_ring_rollback), since every slot they overwrote held a
 * position older than the window that remains (after an earlier rollback the exact depth can be
 * smaller; see wmtp_ring_rollback). slack = 0 is the compact ring of the Windowed-MTP abstract
 * (last sentence). */
typedef struct wmtp_kv {
  void* k;          /* device [batch][n_kv_heads][capacity][head_dim] */
  void* v;          /* device [batch][n_kv_heads][capacity][head_dim] */
  int32_t* pos;     /* device [batch][capacity]: position held by each slot, or NULL */
  int32_t* seq_len; /* device [batch]: tokens appended so far */
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t sink;
  int32_t window;
  int32_t dtype; /* wmtp_dtype */
} wmtp_kv;

/* Append n_new tokens to every sequence (the k_new/v_new rows of sequence b get positions
 * seq_len[b] .. seq_len[b] + n_new - 1), then seq_len[b] += n_new, all on `stream`.
 * For each token, K and V of every KV head are copied bit for bit into slot(p), and pos[b][slot]
 * is set to p when pos is not NULL. In a ring, only the tokens that are still held after the
 * append are written (sinks, and the last capacity - sink positions), so a bulk append of any size
 * writes each slot at most once. In a contiguous cache, tokens whose position would reach `capacity` are
 * not written (seq_len still advances; the caller's contract is seq_len[b] + n_new <= capacity,
 * which the device cannot report).
 * Errors: INVALID_ARG (null pointers, n_new < 0, bad descriptor), UNSUPPORTED (dtype, head_dim),
 * CAPACITY (contiguous cache with n_new > capacity), HIP. n_new = 0 is a no-op returning WMTP_OK. */
int wmtp_ring_append(const wmtp_kv* cache, const void* k_new, const void* v_new, int32_t n_new,
                     void* stream);

/* Windowed-MTP draft step (abstract, fifth sentence): one query token per sequence (q is
 * [batch][1][n_q_heads][head_dim]) attends its ring's sink positions {p < sink} and the last
 * `window` positions {n_b - window <= p < n_b}, each once, n_b = seq_len[b]. Without slack these are
 * exactly the occupied slots 0..min(n_b, capacity)-1; with slack, the slots holding older positions
 * are skipped. `ring` must be a ring (window >= 1). out is [batch][1][n_q_heads][head_dim] float32; lse (nullable) [batch][1][n_q_heads].
 * A sequence with seq_len[b] <= 0 gets out = 0 and lse = -inf.
 * ws: device workspace of at least
 *   wmtp_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, 1, capacity) bytes.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
int wmtp_draft_attn_windowed(const wmtp_kv* ring, const void* q, int32_t n_q_heads, float sm_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* A whole Windowed-MTP draft step in one call: exactly wmtp_ring_append(ring, k_new, v_new, 1)
 * followed by wmtp_draft_attn_windowed(ring, q, ...) (abstract, fourth and fifth sentences: each
 * draft step adds its token, then the draft attends sinks + window), with the same results, ring
 * bytes, tags and seq_len. k_new/v_new are [batch][1][n_kv_heads][head_dim]. When one row block
 * holds the query heads of a KV head (n_q_heads / n_kv_heads <= 16) it runs as two launches instead
 * of three: the attention kernel reads the new token from k_new/v_new while storing it, and the
 * merge advances seq_len. Workspace and errors as for wmtp_draft_attn_windowed. */
int wmtp_draft_step_windowed(const wmtp_kv* ring, const void* k_new, const void* v_new,
                             const void* q, int32_t n_q_heads, float sm_scale, float* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream);

/* The native full-context draft step in one call: wmtp_ring_append(cache, k_new, v_new, 1) then
 * wmtp_draft_attn_full(cache, q, ..., max_seq_len, ...); max_seq_len must bound the lengths after
 * the append. Same fusion as wmtp_draft_step_windowed. */
int wmtp_draft_step_full(const wmtp_kv* cache, const void* k_new, const void* v_new, const void* q,
                         int32_t n_q_heads, float sm_scale, int32_t max_seq_len, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream);

/* Native full-context draft step: one query token per sequence attends every cached position
 * 0..n_b-1 of a contiguous cache (window == 0), n_b = min(seq_len[b], capacity). max_seq_len is a
 * host-side upper bound on every seq_len[b] (1 <= max_seq_len <= capacity), used only to size the
 * launch; positions at or beyond max_seq_len are never read. out/lse as for the windowed call.
 * ws: at least wmtp_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, 1, max_seq_len).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
int wmtp_draft_attn_full(const wmtp_kv* cache, const void* q, int32_t n_q_heads, float sm_scale,
                         int32_t max_seq_len, float* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* Target verification of m draft candidates with full attention: the candidates are the last m
 * cached positions n_b-m .. n_b-1 of a contiguous cache (window == 0), and candidate j attends
 * positions 0 .. n_b-m+j (the prefix plus candidates 0..j). q is [batch][m][n_q_heads][head_dim];
 * out [batch][m][n_q_heads][head_dim] float32; lse (nullable) [batch][m][n_q_heads]. A candidate
 * with no visible position (n_b-m+j < 0) gets out = 0 and lse = -inf. 1 <= m <= 16.
 * ws: at least wmtp_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, m, max_seq_len).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
int wmtp_verify_attn(const wmtp_kv* cache, const void* q, int32_t m, int32_t n_q_heads,
                     float sm_scale, int32_t max_seq_len, float* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/* MASW-style draft step (MASW page, section 4.1: the working memory is the sink tokens, an exact
 * local window and compressed memory slots): one query token per sequence attends its ring's sinks
 * and last `window` positions (exactly as wmtp_draft_attn_windowed) together with memory slots
 * 0 .. slots->seq_len[b]-1 of `slots`, a contiguous cache (window = 0) holding one K/V row per
 * materialised slot, appended by the caller (wmtp_ring_append) as slots are made; how a slot is
 * made from history is not this library's business. Both caches must share batch, n_kv_heads,
 * head_dim and dtype. max_slots is a host bound on every slots->seq_len[b]
 * (1 <= max_slots <= slots->capacity), used only to size the launch. The two reads write one set
 * of split partials and one log-sum-exp merge combines them, so the result is softmax attention
 * over the union. out/lse as for the windowed call.
 * ws: at least wmtp_masw_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, ring->capacity,
 * max_slots) bytes. Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
int wmtp_draft_attn_masw(const wmtp_kv* ring, const wmtp_kv* slots, const void* q,
                         int32_t n_q_heads, float sm_scale, int32_t max_slots, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of wmtp_draft_attn_masw; 0 for sizes it rejects. */
size_t wmtp_masw_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t ring_capacity, int32_t max_slots);

/* Discard the newest n_drop[b] tokens of every sequence b after a rejected speculation (the MASW
 * page, section 4.3: rejected speculative local KV is discarded). n_drop is device memory [batch],
 * typically written by wmtp_greedy_accept on the same stream. The count is clamped on the device:
 * to [0, seq_len[b]] for a contiguous cache (which overwrites nothing), and for a ring to the
 * largest d <= min(n_drop[b], seq_len[b], slack) after which every position the windowed draft
 * attends (the sinks and the last `window` of the seq_len[b] - d that remain) is still held in its
 * slot. Without earlier rollbacks that is min(n_drop[b], seq_len[b], slack); after a rollback,
 * tokens appended again reuse the slots of the discarded ones while the older window slots they
 * overwrote stay lost, so a second rollback deeper than what was appended since can be cut
 * shorter. A ring's depth is read from the pos tags, so a ring with slack needs pos (INVALID_ARG
 * otherwise), kept by the library's appends. The slots of the discarded positions get pos = -1
 * (when pos is not NULL; positions at or past a contiguous cache's capacity have no slot), then
 * seq_len[b] shrinks by the count. K/V bytes are left as they are (no call reads them until a
 * later append overwrites them). Errors: INVALID_ARG (null or misaligned n_drop, a ring with
 * slack and no pos, bad descriptor), UNSUPPORTED, HIP. */
int wmtp_ring_rollback(const wmtp_kv* cache, const int32_t* n_drop, void* stream);

/* Greedy verification of k draft tokens per sequence from the target's logits (the target's
 * standard accept/reject rule under greedy decoding; MASW page, sections 1 and 4.3).
 *   logits       device [batch][k+1][vocab], dtype WMTP_F32 or WMTP_BF16 (element-aligned): row i
 *                scores the token after the prefix and the first i drafts. No NaN entries.
 *   draft_tokens device int32 [batch][k] (may be NULL when k = 0)
 *   choice       device int32 [batch][k+1]: argmax of every row (the lowest index on ties)
 *   n_accept     device int32 [batch]: a = the number of leading drafts equal to choice[b][i]
 *   next_token   device int32 [batch]: choice[b][a] (the correction, or the bonus token if a = k)
 *   n_drop       device int32 [batch]: k - a (the draft tokens a rollback should discard)
 * 0 <= k <= 63, batch*(k+1) <= 65535, vocab >= 1. ws: device, 256-byte aligned, at least
 * wmtp_accept_workspace_bytes(batch, k, vocab) bytes. Errors: INVALID_ARG, UNSUPPORTED (dtype),
 * WORKSPACE, HIP. */
int wmtp_greedy_accept(const void* logits, int32_t dtype, int32_t batch, int32_t k, int32_t vocab,
                       const int32_t* draft_tokens, int32_t* choice, int32_t* n_accept,
                       int32_t* next_token, int32_t* n_drop, void* ws, size_t ws_bytes,
                       void* stream);

/* Workspace bytes of wmtp_greedy_accept (per-chunk maxima); 0 for arguments it rejects. */
size_t wmtp_accept_workspace_bytes(int32_t batch, int32_t k, int32_t vocab);

/* The target's append + verification in one call: wmtp_ring_append(cache, k_new, v_new, m) then
 * wmtp_verify_attn(cache, q, m, ...); k_new/v_new are [batch][m][n_kv_heads][head_dim] and
 * max_seq_len must bound the lengths after the append. When the cooperative kernel runs the
 * verification (more query rows per KV head, m * n_q_heads / n_kv_heads, than the key-split
 * kernel takes: 16 for m = 1, else 48, or 32 for bf16 at head_dim 256 and fp32 at 128, 16 for fp32
 * at 256) it reads
 * the candidates from k_new/v_new while storing them and the merge advances seq_len (two launches
 * instead of three); otherwise the append runs first. Results, cache bytes and lengths equal the
 * two calls. Errors as for wmtp_verify_attn. */
int wmtp_verify_step(const wmtp_kv* cache, const void* k_new, const void* v_new, const void* q,
                     int32_t m, int32_t n_q_heads, float sm_scale, int32_t max_seq_len, float* out,
                     float* lse, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): exactly wmtp_draft_step_windowed(ring, k_new, v_new,
 * q, n_q_heads, sm_scale, out, lse, ws, ws_bytes, stream), with the same kernels, results, ring
 * bytes, tags and seq_len, but with no workspace argument: the split-K partials go to a static
 * device array of WMTP_NOALLOC_SCRATCH_BYTES that the library's code object holds on every GPU it
 * runs on until the process ends. The call allocates and frees nothing. Its device address is
 * looked up (hipGetSymbolAddress) on the first call on each device, so the current device must be
 * the one `stream` belongs to. Every call on a GPU shares that GPU's array: calls that may overlap
 * on one GPU (other streams, other host threads) race and must be serialised by the caller. The
 * partials are written in full before they are read, so the array needs no clearing.
 * Errors: as for wmtp_draft_step_windowed; WMTP_ERR_WORKSPACE when the step needs more than
 * WMTP_NOALLOC_SCRATCH_BYTES (wmtp_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
 * 1, capacity) is the need); WMTP_ERR_HIP when the array's address cannot be obtained. */
#define WMTP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int wmtp_draft_step_windowed_noalloc(const wmtp_kv* ring, const void* k_new, const void* v_new,
                                     const void* q, int32_t n_q_heads, float sm_scale, float* out,
                                     float* lse, void* stream);

/* Workspace bytes an attention call with these sizes needs (split-K partial results). Pass
 * m = 1 for draft steps and max_seq_len = capacity for the windowed call. Depends only on its
 * arguments (not on the device). Returns 0 for arguments no attention call accepts. */
size_t wmtp_attn_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t m, int32_t max_seq_len);

/* Static, human-readable name of a wmtp_status value (never NULL). */
const char* wmtp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* WMTP_H */

// abi.hip -- the extern "C" entry points of libwmtp.so (declared and documented in wmtp.h):
// host-side validation, split planning and launches. No allocation and no synchronisation. The
// only state is the per-device address of the allocation-free entry point's static scratch
// array (below), looked up once per device.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "wmtp_internal.h"

namespace {

using wmtp::SplitPlan;

constexpr size_t kAlign = 256;
constexpr int kMaxAcceptK = 63;  // draft tokens per greedy verification

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t plan_bytes(const SplitPlan& p) {
  return round_up(p.ws_o_floats * sizeof(float), kAlign) + p.ws_ml_floats * sizeof(float);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int dtype) { return dtype == WMTP_BF16 ? 2 : 4; }

// Checks shared by every call. Returns WMTP_OK or the status to report.
int check_kv(const wmtp_kv* c) {
  if (!c) return WMTP_ERR_INVALID_ARG;
  if (c->dtype != WMTP_F32 && c->dtype != WMTP_BF16) return WMTP_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return WMTP_ERR_UNSUPPORTED;
  if (!c->k || !c->v || !c->seq_len) return WMTP_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->capacity < 1) return WMTP_ERR_INVALID_ARG;
  if (c->batch > 65535) return WMTP_ERR_INVALID_ARG;  // one grid row per sequence in the appends
  if (c->capacity > wmtp::kMaxCapacity) return WMTP_ERR_CAPACITY;
  if (c->sink < 0 || c->window < 0) return WMTP_ERR_INVALID_ARG;
  if (c->window >= 1) {
    // a ring: S sinks, W attended window slots and capacity - S - W >= 0 slack slots
    if ((long long)c->sink + c->window > c->capacity) return WMTP_ERR_INVALID_ARG;
  } else if (c->sink != c->capacity) {
    return WMTP_ERR_INVALID_ARG;
  }
  if (!aligned(c->k, 16) || !aligned(c->v, 16) || !aligned(c->seq_len, 4)) return WMTP_ERR_INVALID_ARG;
  if (c->pos && !aligned(c->pos, 4)) return WMTP_ERR_INVALID_ARG;
  return WMTP_OK;
}

int append_call(const wmtp_kv* cache, const void* k_new, const void* v_new, int32_t n_new,
                void* stream) {
  int st = check_kv(cache);
  if (st != WMTP_OK) return st;
  if (n_new < 0) return WMTP_ERR_INVALID_ARG;
  if (n_new == 0) return WMTP_OK;
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return WMTP_ERR_INVALID_ARG;
  if (cache->window == 0 && n_new > cache->capacity) return WMTP_ERR_CAPACITY;
  wmtp::AppendArgs a;
  a.k = cache->k;
  a.v = cache->v;
  a.pos = cache->pos;
  a.seq_len = cache->seq_len;
  a.k_new = k_new;
  a.v_new = v_new;
  a.batch = cache->batch;
  a.n_kv_heads = cache->n_kv_heads;
  a.head_dim = cache->head_dim;
  a.capacity = cache->capacity;
  a.sink = cache->sink;
  a.window = cache->window == 0 ? 0 : cache->capacity - cache->sink;  // physical window
  a.n_new = n_new;
  a.elem_bytes = elem_bytes(cache->dtype);
  hipError_t e = wmtp::launch_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}


// new_k/new_v (nullable): a fused draft step appends one token per sequence first. The split
// kernel does both in one launch; a cooperative-kernel shape appends with the append kernel first.
int attention_call(const wmtp_kv* c, const void* q, int m, int n_q_heads, float sm_scale,
                   int limit, int mode, float* out, float* lse, void* ws, size_t ws_bytes,
                   void* stream, const void* new_k = nullptr, const void* new_v = nullptr) {
  if (!q || !out) return WMTP_ERR_INVALID_ARG;
  if (new_k && (!new_v || !aligned(new_k, 16) || !aligned(new_v, 16))) return WMTP_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4))) return WMTP_ERR_INVALID_ARG;
  if (n_q_heads < c->n_kv_heads || n_q_heads % c->n_kv_heads) return WMTP_ERR_INVALID_ARG;
  if (!isfinite(sm_scale)) return WMTP_ERR_INVALID_ARG;
  SplitPlan plan;
  if (!wmtp::make_plan_for(c->batch, n_q_heads, c->n_kv_heads, c->head_dim, m, limit, c->dtype,
                           &plan))
    return WMTP_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < plan_bytes(plan)) return WMTP_ERR_WORKSPACE;

  wmtp::AttnArgs a{};  // every field zero (no fused append, no partial offset) unless set
  a.q = q;
  a.k = c->k;
  a.v = c->v;
  a.seq_len = c->seq_len;
  a.out = out;
  a.lse = lse;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                     round_up(plan.ws_o_floats * sizeof(float), kAlign));
  a.batch = c->batch;
  a.n_kv_heads = c->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.head_dim = c->head_dim;
  a.m = m;
  a.capacity = c->capacity;
  a.limit = limit;
  a.mode = mode;
  a.sm_scale = sm_scale;
  a.sink = c->sink;
  a.window = c->window;
  a.wphys = c->window >= 1 ? c->capacity - c->sink : 0;
  a.part_stride = plan.n_splits;
  a.part_offset = 0;
  if (new_k) {
    // one-launch forms: the split kernel with one new token (draft steps), the cooperative kernel
    // on a contiguous cache (verification); anything else appends first
    const bool fused = plan.coop ? (mode == wmtp::kModeVerify) : (m == 1);
    if (fused) {
      a.new_k = new_k;
      a.new_v = new_v;
      a.pos = c->pos;
    } else {
      const int st = append_call(c, new_k, new_v, m, stream);
      if (st != WMTP_OK) return st;
    }
  }
  hipError_t e = wmtp::launch_attention(a, plan, c->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

// Plans of the two reads of a MASW draft step (the ring's sinks + window, the memory slots). Both
// have the same row chunking (one query token, same heads and dtype); their partials share one
// merge. Returns false when no call accepts the sizes.
bool masw_plans(const wmtp_kv* ring, int n_q_heads, int max_slots, SplitPlan* pr, SplitPlan* ps) {
  return wmtp::make_plan_for(ring->batch, n_q_heads, ring->n_kv_heads, ring->head_dim, 1,
                             ring->capacity, ring->dtype, pr) &&
         wmtp::make_plan_for(ring->batch, n_q_heads, ring->n_kv_heads, ring->head_dim, 1,
                             max_slots, ring->dtype, ps);
}

size_t masw_bytes(const SplitPlan& pr, const SplitPlan& ps) {
  SplitPlan both = pr;
  both.n_splits = pr.n_splits + ps.n_splits;
  both.ws_o_floats = pr.ws_o_floats + ps.ws_o_floats;
  both.ws_ml_floats = pr.ws_ml_floats + ps.ws_ml_floats;
  return plan_bytes(both);
}

// ---- scratch of the allocation-free windowed draft step (wmtp_draft_step_windowed_noalloc)
// Device memory of the split-K partials, part of the library's code object: every GPU the library
// runs on holds its own copy from the first use of the library on it until the process ends.
// Host code must not pass `scratch` itself to a kernel (in host code the name is a host-side
// stand-in, not a device address): its device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_addr.
constexpr size_t kScratchBytes = WMTP_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];

// The current device's scratch address (looked up on the first call on that device), or NULL
// when the HIP runtime cannot report it.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_addr[dev] = p;
  }
  return scratch_addr[dev];
}

}  // namespace

extern "C" {

int wmtp_draft_step_windowed_noalloc(const wmtp_kv* ring, const void* k_new, const void* v_new,
                                     const void* q, int32_t n_q_heads, float sm_scale, float* out,
                                     float* lse, void* stream) {
  int st = check_kv(ring);
  if (st != WMTP_OK) return st;
  if (ring->window < 1 || !k_new || !v_new) return WMTP_ERR_INVALID_ARG;
  // the partials this step needs must fit the static scratch (checked before any lookup)
  const size_t need = wmtp_attn_workspace_bytes(ring->batch, n_q_heads, ring->n_kv_heads,
                                                ring->head_dim, 1, ring->capacity);
  if (need == 0) return WMTP_ERR_INVALID_ARG;
  if (need > kScratchBytes) return WMTP_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return WMTP_ERR_HIP;
  // the partials are written in full before the merge reads them: nothing must start at zero
  return attention_call(ring, q, 1, n_q_heads, sm_scale, ring->capacity, wmtp::kModeWindowed, out,
                        lse, ws, kScratchBytes, stream, k_new, v_new);
}

int wmtp_ring_append(const wmtp_kv* cache, const void* k_new, const void* v_new, int32_t n_new,
                     void* stream) {
  return append_call(cache, k_new, v_new, n_new, stream);
}

int wmtp_draft_step_windowed(const wmtp_kv* ring, const void* k_new, const void* v_new,
                             const void* q, int32_t n_q_heads, float sm_scale, float* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_kv(ring);
  if (st != WMTP_OK) return st;
  if (ring->window < 1 || !k_new || !v_new) return WMTP_ERR_INVALID_ARG;
  return attention_call(ring, q, 1, n_q_heads, sm_scale, ring->capacity, wmtp::kModeWindowed, out,
                        lse, ws, ws_bytes, stream, k_new, v_new);
}

int wmtp_draft_step_full(const wmtp_kv* cache, const void* k_new, const void* v_new, const void* q,
                         int32_t n_q_heads, float sm_scale, int32_t max_seq_len, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_kv(cache);
  if (st != WMTP_OK) return st;
  if (cache->window != 0 || !k_new || !v_new) return WMTP_ERR_INVALID_ARG;
  if (max_seq_len < 1 || max_seq_len > cache->capacity) return WMTP_ERR_INVALID_ARG;
  return attention_call(cache, q, 1, n_q_heads, sm_scale, max_seq_len, wmtp::kModeFull, out, lse,
                        ws, ws_bytes, stream, k_new, v_new);
}


int wmtp_draft_attn_windowed(const wmtp_kv* ring, const void* q, int32_t n_q_heads, float sm_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_kv(ring);
  if (st != WMTP_OK) return st;
  if (ring->window < 1) return WMTP_ERR_INVALID_ARG;
  return attention_call(ring, q, 1, n_q_heads, sm_scale, ring->capacity, wmtp::kModeWindowed, out,
                        lse, ws, ws_bytes, stream);
}

int wmtp_draft_attn_full(const wmtp_kv* cache, const void* q, int32_t n_q_heads, float sm_scale,
                         int32_t max_seq_len, float* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  int st = check_kv(cache);
  if (st != WMTP_OK) return st;
  if (cache->window != 0) return WMTP_ERR_INVALID_ARG;
  if (max_seq_len < 1 || max_seq_len > cache->capacity) return WMTP_ERR_INVALID_ARG;
  return attention_call(cache, q, 1, n_q_heads, sm_scale, max_seq_len, wmtp::kModeFull, out, lse,
                        ws, ws_bytes, stream);
}

int wmtp_verify_attn(const wmtp_kv* cache, const void* q, int32_t m, int32_t n_q_heads,
                     float sm_scale, int32_t max_seq_len, float* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_kv(cache);
  if (st != WMTP_OK) return st;
  if (cache->window != 0) return WMTP_ERR_INVALID_ARG;
  if (m < 1 || m > wmtp::kMaxM) return WMTP_ERR_INVALID_ARG;
  if (max_seq_len < 1 || max_seq_len > cache->capacity) return WMTP_ERR_INVALID_ARG;
  return attention_call(cache, q, m, n_q_heads, sm_scale, max_seq_len, wmtp::kModeVerify, out, lse,
                        ws, ws_bytes, stream);
}

int wmtp_draft_attn_masw(const wmtp_kv* ring, const wmtp_kv* slots, const void* q,
                         int32_t n_q_heads, float sm_scale, int32_t max_slots, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_kv(ring);
  if (st != WMTP_OK) return st;
  st = check_kv(slots);
  if (st != WMTP_OK) return st;
  if (ring->window < 1 || slots->window != 0) return WMTP_ERR_INVALID_ARG;
  if (slots->batch != ring->batch || slots->n_kv_heads != ring->n_kv_heads ||
      slots->head_dim != ring->head_dim || slots->dtype != ring->dtype)
    return WMTP_ERR_INVALID_ARG;
  if (max_slots < 1 || max_slots > slots->capacity) return WMTP_ERR_INVALID_ARG;
  if (!q || !out) return WMTP_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4))) return WMTP_ERR_INVALID_ARG;
  if (n_q_heads < ring->n_kv_heads || n_q_heads % ring->n_kv_heads) return WMTP_ERR_INVALID_ARG;
  if (!isfinite(sm_scale)) return WMTP_ERR_INVALID_ARG;
  SplitPlan pr, ps;
  if (!masw_plans(ring, n_q_heads, max_slots, &pr, &ps)) return WMTP_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < masw_bytes(pr, ps)) return WMTP_ERR_WORKSPACE;

  const int total = pr.n_splits + ps.n_splits;
  const size_t o_floats = pr.ws_o_floats + ps.ws_o_floats;
  wmtp::AttnArgs a{};  // every field zero (no fused append, no partial offset) unless set
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up(o_floats * sizeof(float), kAlign));
  a.batch = ring->batch;
  a.n_kv_heads = ring->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.head_dim = ring->head_dim;
  a.m = 1;
  a.sm_scale = sm_scale;
  a.part_stride = total;
  // read 1: the ring's sinks and last `window` positions (partials 0 .. pr.n_splits-1)
  a.k = ring->k;
  a.v = ring->v;
  a.seq_len = ring->seq_len;
  a.capacity = ring->capacity;
  a.limit = ring->capacity;
  a.mode = wmtp::kModeWindowed;
  a.sink = ring->sink;
  a.window = ring->window;
  a.wphys = ring->capacity - ring->sink;
  a.part_offset = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = wmtp::launch_partials(a, pr, ring->dtype, s);
  if (e != hipSuccess) return WMTP_ERR_HIP;
  // read 2: memory slots 0 .. slots->seq_len[b]-1 (partials pr.n_splits .. total-1)
  wmtp::AttnArgs b = a;
  b.k = slots->k;
  b.v = slots->v;
  b.seq_len = slots->seq_len;
  b.capacity = slots->capacity;
  b.limit = max_slots;
  b.mode = wmtp::kModeFull;
  b.sink = slots->sink;
  b.window = 0;
  b.wphys = 0;
  b.part_offset = pr.n_splits;
  e = wmtp::launch_partials(b, ps, ring->dtype, s);
  if (e != hipSuccess) return WMTP_ERR_HIP;
  e = wmtp::launch_merge(a, pr, total, s);
  return e == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

int wmtp_verify_step(const wmtp_kv* cache, const void* k_new, const void* v_new, const void* q,
                     int32_t m, int32_t n_q_heads, float sm_scale, int32_t max_seq_len, float* out,
                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_kv(cache);
  if (st != WMTP_OK) return st;
  if (cache->window != 0 || !k_new || !v_new) return WMTP_ERR_INVALID_ARG;
  if (m < 1 || m > wmtp::kMaxM) return WMTP_ERR_INVALID_ARG;
  if (max_seq_len < 1 || max_seq_len > cache->capacity) return WMTP_ERR_INVALID_ARG;
  return attention_call(cache, q, m, n_q_heads, sm_scale, max_seq_len, wmtp::kModeVerify, out, lse,
                        ws, ws_bytes, stream, k_new, v_new);
}

size_t wmtp_masw_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t ring_capacity, int32_t max_slots) {
  size_t best = 0;
  const int dtypes[2] = {WMTP_F32, WMTP_BF16};
  for (int dt : dtypes) {
    wmtp_kv r = {};
    r.batch = batch;
    r.n_kv_heads = n_kv_heads;
    r.head_dim = head_dim;
    r.capacity = ring_capacity;
    r.dtype = dt;
    SplitPlan pr, ps;
    if (!masw_plans(&r, n_q_heads, max_slots, &pr, &ps)) return 0;
    const size_t bytes = masw_bytes(pr, ps);
    if (bytes > best) best = bytes;
  }
  return best;
}

int wmtp_ring_rollback(const wmtp_kv* cache, const int32_t* n_drop, void* stream) {
  int st = check_kv(cache);
  if (st != WMTP_OK) return st;
  if (!n_drop || !aligned(n_drop, 4)) return WMTP_ERR_INVALID_ARG;
  // a ring's exact rollback depth is read from its position tags
  if (cache->window >= 1 && cache->capacity - cache->sink - cache->window > 0 && !cache->pos)
    return WMTP_ERR_INVALID_ARG;
  wmtp::RollbackArgs a;
  a.pos = cache->pos;
  a.seq_len = cache->seq_len;
  a.n_drop = n_drop;
  a.batch = cache->batch;
  a.capacity = cache->capacity;
  a.sink = cache->sink;
  a.window = cache->window == 0 ? 0 : cache->capacity - cache->sink;
  a.slack = cache->window == 0 ? 0 : cache->capacity - cache->sink - cache->window;
  hipError_t e = wmtp::launch_rollback(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

size_t wmtp_accept_workspace_bytes(int32_t batch, int32_t k, int32_t vocab) {
  if (batch < 1 || k < 0 || k > kMaxAcceptK || vocab < 1) return 0;
  const size_t chunks = ((size_t)vocab + wmtp::kAcceptChunk - 1) / wmtp::kAcceptChunk;
  const size_t entries = (size_t)batch * (k + 1) * chunks;
  return round_up(entries * sizeof(float), kAlign) + entries * sizeof(int32_t);
}

int wmtp_greedy_accept(const void* logits, int32_t dtype, int32_t batch, int32_t k, int32_t vocab,
                       const int32_t* draft_tokens, int32_t* choice, int32_t* n_accept,
                       int32_t* next_token, int32_t* n_drop, void* ws, size_t ws_bytes,
                       void* stream) {
  if (dtype != WMTP_F32 && dtype != WMTP_BF16) return WMTP_ERR_UNSUPPORTED;
  if (batch < 1 || k < 0 || k > kMaxAcceptK || vocab < 1) return WMTP_ERR_INVALID_ARG;
  if ((size_t)batch * (k + 1) > 65535) return WMTP_ERR_INVALID_ARG;  // one grid row each
  if (!logits || !aligned(logits, elem_bytes(dtype))) return WMTP_ERR_INVALID_ARG;
  if (k > 0 && (!draft_tokens || !aligned(draft_tokens, 4))) return WMTP_ERR_INVALID_ARG;
  if (!choice || !n_accept || !next_token || !n_drop) return WMTP_ERR_INVALID_ARG;
  if (!aligned(choice, 4) || !aligned(n_accept, 4) || !aligned(next_token, 4) || !aligned(n_drop, 4))
    return WMTP_ERR_INVALID_ARG;
  const size_t need = wmtp_accept_workspace_bytes(batch, k, vocab);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return WMTP_ERR_WORKSPACE;
  wmtp::AcceptArgs a;
  a.logits = logits;
  a.draft = draft_tokens;
  a.choice = choice;
  a.n_accept = n_accept;
  a.next_token = next_token;
  a.n_drop = n_drop;
  a.batch = batch;
  a.k = k;
  a.vocab = vocab;
  a.chunks = (vocab + wmtp::kAcceptChunk - 1) / wmtp::kAcceptChunk;
  a.dtype = dtype;
  const size_t entries = (size_t)batch * (k + 1) * a.chunks;
  a.ws_val = static_cast<float*>(ws);
  a.ws_idx = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                        round_up(entries * sizeof(float), kAlign));
  hipError_t e = wmtp::launch_accept(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

size_t wmtp_attn_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t m, int32_t max_seq_len) {
  // the largest need over the supported dtypes, so one size serves every cache
  size_t best = 0;
  const int dtypes[2] = {WMTP_F32, WMTP_BF16};
  for (int dt : dtypes) {
    SplitPlan p;
    if (!wmtp::make_plan_for(batch, n_q_heads, n_kv_heads, head_dim, m, max_seq_len, dt, &p))
      return 0;
    const size_t bytes = plan_bytes(p);
    if (bytes > best) best = bytes;
  }
  return best;
}

const char* wmtp_status_string(int status) {
  switch (status) {
    case WMTP_OK: return "WMTP_OK";
    case WMTP_ERR_INVALID_ARG: return "WMTP_ERR_INVALID_ARG: invalid argument";
    case WMTP_ERR_UNSUPPORTED: return "WMTP_ERR_UNSUPPORTED: dtype or head_dim not implemented";
    case WMTP_ERR_CAPACITY: return "WMTP_ERR_CAPACITY: request exceeds the cache capacity";
    case WMTP_ERR_WORKSPACE: return "WMTP_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case WMTP_ERR_HIP: return "WMTP_ERR_HIP: HIP launch error";
    default: return "unknown wmtp status";
  }
}

}  // extern "C"

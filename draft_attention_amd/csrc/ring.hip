// ring.hip -- append of new tokens' K/V into a compact ring buffer or a contiguous cache.
//
// The compact ring buffer holds what the Windowed-MTP draft reads and nothing else (Windowed-MTP
// abstract, last sentence: the unread draft KV is reclaimed by a compact ring buffer): S pinned
// sink slots and W window slots that wrap. Position p lives in slot p if p < S, else in slot
// S + (p - S) mod W. A contiguous cache is the same map with W = 0 (slot = p).
//
// Only survivors are written: of the n_new tokens appended at positions n .. n+n_new-1 of a ring,
// a token is still held afterwards iff it is a sink (p < S) or one of the last W positions
// (p >= n + n_new - W); any other token would be overwritten within the same append. So a bulk
// append never writes one slot twice, and the workgroups of a launch never race on a slot.
//
// A ring may carry slack window slots beyond the W the draft attends (capacity = S + W + slack):
// appends then wrap over W + slack slots (the `window` these kernels receive is that physical
// window), and the newest `slack` tokens can be discarded again exactly (rollback_kernel): every
// slot they overwrote held a position older than the W-token window that remains.
//
// seq_len[b] is read by every thread that computes slots and advanced by n_new. When one workgroup
// handles a whole sequence it advances seq_len itself after a barrier (one launch); when a bulk
// append is spread over many workgroups, a second one-wavefront kernel advances it after the copy.

#include "wmtp_internal.h"

namespace wmtp {
namespace {

struct Survivors {
  int64_t n;       // tokens present before the append (>= 0)
  int64_t first;   // survivors u < first are tokens t = u (sinks appended now)
  int64_t second;  // survivors u >= first are tokens t = second + (u - first)
  int64_t count;   // number of survivors
};

__device__ __forceinline__ Survivors survivors_of(int64_t n, int sink, int window, int capacity,
                                                  int n_new) {
  Survivors s;
  s.n = n;
  if (window == 0) {
    // contiguous cache: every token below capacity
    const int64_t room = capacity > n ? capacity - n : 0;
    s.first = 0;
    s.second = 0;
    s.count = n_new < room ? n_new : room;
    return s;
  }
  int64_t a = sink - n;  // tokens of this append that are sinks
  if (a < 0) a = 0;
  if (a > n_new) a = n_new;
  int64_t w0 = (int64_t)n_new - window;  // first token that is among the last W
  if (w0 < a) w0 = a;
  s.first = a;
  s.second = w0;
  s.count = a + (n_new - w0);
  return s;
}

__device__ __forceinline__ int64_t slot_of(int64_t p, int sink, int window) {
  if (window == 0 || p < sink) return p;
  return sink + (p - sink) % window;
}

// Copy the survivors' rows of sequence b; threads of the x/y grid share the work.
__device__ __forceinline__ void copy_rows(const AppendArgs& a, int b, const Survivors& sv,
                                          int64_t tid, int64_t nthreads) {
  const int chunks = a.head_dim * a.elem_bytes / 16;  // 16-byte pieces per row
  const int64_t total = sv.count * a.n_kv_heads * chunks;
  for (int64_t i = tid; i < total; i += nthreads) {
    const int c = (int)(i % chunks);
    const int64_t r = i / chunks;
    const int h = (int)(r % a.n_kv_heads);
    const int64_t u = r / a.n_kv_heads;
    const int64_t t = u < sv.first ? u : sv.second + (u - sv.first);
    const int64_t p = sv.n + t;
    const int64_t slot = slot_of(p, a.sink, a.window);
    const size_t src = (((size_t)b * a.n_new + t) * a.n_kv_heads + h) * chunks + c;
    const size_t dst = (((size_t)b * a.n_kv_heads + h) * a.capacity + slot) * chunks + c;
    reinterpret_cast<uint4*>(a.k)[dst] = reinterpret_cast<const uint4*>(a.k_new)[src];
    reinterpret_cast<uint4*>(a.v)[dst] = reinterpret_cast<const uint4*>(a.v_new)[src];
    if (a.pos && h == 0 && c == 0) a.pos[(size_t)b * a.capacity + slot] = (int32_t)p;
  }
}

__device__ __forceinline__ int64_t present(const int32_t* seq_len, int b) {
  const int32_t n = seq_len[b];
  return n > 0 ? n : 0;
}

// One workgroup per sequence: copy, barrier, then advance seq_len (no other workgroup reads it).
__global__ __launch_bounds__(256) void append_fused_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int64_t n = present(a.seq_len, b);
  const Survivors sv = survivors_of(n, a.sink, a.window, a.capacity, a.n_new);
  copy_rows(a, b, sv, threadIdx.x, blockDim.x);
  __syncthreads();  // every thread has read seq_len[b] before it changes
  if (threadIdx.x == 0) {
    const int64_t next = n + a.n_new;
    a.seq_len[b] = (int32_t)(next > 0x7fffffffLL ? 0x7fffffffLL : next);
  }
}

// Bulk copy over many workgroups per sequence; seq_len is only read here.
__global__ __launch_bounds__(256) void append_copy_kernel(AppendArgs a) {
  const int b = blockIdx.y;
  const int64_t n = present(a.seq_len, b);
  const Survivors sv = survivors_of(n, a.sink, a.window, a.capacity, a.n_new);
  copy_rows(a, b, sv, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
            (int64_t)gridDim.x * blockDim.x);
}

__global__ __launch_bounds__(64) void append_bump_kernel(int32_t* seq_len, int batch, int n_new) {
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int64_t next = present(seq_len, b) + n_new;
    seq_len[b] = (int32_t)(next > 0x7fffffffLL ? 0x7fffffffLL : next);
  }
}

// Deepest exact rollback of a ring (one wavefront, uniform result): the largest d <= d0 such
// that the draft's attended set with n - d tokens present -- the sinks and the last W positions
// -- is still held. Sinks are never overwritten, so only the oldest window position
// q = max(S, n - d - W) has to be checked: the window positions still held form the run
// [lo, n) (a slot loses position p only when position p + W + slack is appended, and positions
// are appended in order), so q is held iff tag(slot(q)) == q, and that test passes for every d
// up to some depth and fails beyond it. d with n - d <= S leaves sinks only and is always exact.
// Each round tests 64 evenly spaced depths of the open range (one load per lane): depths <= 64
// take one round.
__device__ __forceinline__ int64_t exact_depth(const RollbackArgs& a, int b, int64_t n, int64_t d0) {
  if (d0 <= 0 || n - d0 <= a.sink) return d0 < 0 ? 0 : d0;
  const int lane = threadIdx.x;
  const int attended = a.window - a.slack;
  const int32_t* tags = a.pos + (size_t)b * a.capacity;
  int64_t lo = 0, hi = d0;  // depth lo is exact (0: nothing dropped); the answer is in [lo, hi]
  while (lo < hi) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t c = lo + (int64_t)(lane + 1) * step;  // candidate depth of this lane
    bool ok = false;
    if (c <= hi) {
      const int64_t q0 = n - c - attended;
      const int64_t q = q0 > a.sink ? q0 : (int64_t)a.sink;
      ok = tags[slot_of(q, a.sink, a.window)] == (int32_t)q;
    }
    const uint64_t pass = __ballot(ok);
    const int j = __builtin_ctzll(~pass);  // lanes 0 .. j-1 passed
    const int64_t lo_old = lo;
    if (j > 0) lo = lo_old + (int64_t)j * step;
    if (j < 64 && lo_old + (int64_t)(j + 1) * step <= hi) hi = lo_old + (int64_t)(j + 1) * step - 1;
  }
  return lo;
}

// Discard the newest n_drop[b] tokens of sequence b, clamped to [0, n] for a contiguous cache and
// to the deepest exact rollback within [0, min(n, slack)] for a ring (exact_depth): the tags of
// their slots become -1 and seq_len[b] shrinks. One wavefront per sequence; every lane reads
// seq_len[b] before lane 0 changes it.
__global__ __launch_bounds__(64) void rollback_kernel(RollbackArgs a) {
  const int b = blockIdx.x;
  const int64_t n = present(a.seq_len, b);
  int64_t d = a.n_drop[b];
  const int64_t cap = a.window == 0 ? n : (n < a.slack ? n : (int64_t)a.slack);
  d = d < 0 ? 0 : (d > cap ? cap : d);
  if (a.window != 0) d = exact_depth(a, b, n, d);
  if (a.pos) {
    for (int64_t i = threadIdx.x; i < d; i += blockDim.x) {
      const int64_t p = n - d + i;
      const int64_t slot = slot_of(p, a.sink, a.window);
      if (slot < a.capacity) a.pos[(size_t)b * a.capacity + slot] = -1;  // contiguous: p may pass it
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.seq_len[b] = (int32_t)(n - d);
}

}  // namespace

hipError_t launch_rollback(const RollbackArgs& a, hipStream_t stream) {
  rollback_kernel<<<dim3(a.batch), dim3(64), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  // host-side bound on the survivors of any sequence
  const long long max_surv =
      a.window == 0 ? (a.n_new < a.capacity ? a.n_new : a.capacity)
                    : (a.n_new < (long long)a.sink + a.window ? a.n_new : (long long)a.sink + a.window);
  const long long pieces = max_surv * a.n_kv_heads * (a.head_dim * a.elem_bytes / 16);
  if (pieces <= 256LL * 16) {
    append_fused_kernel<<<dim3(a.batch), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
  }
  long long blocks = (pieces + 256LL * 8 - 1) / (256LL * 8);
  if (blocks > 65535) blocks = 65535;
  append_copy_kernel<<<dim3((unsigned)blocks, a.batch), dim3(256), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  append_bump_kernel<<<dim3(1), dim3(64), 0, stream>>>(a.seq_len, a.batch, a.n_new);
  return hipGetLastError();
}

}  // namespace wmtp

// accept.hip -- greedy verification of k draft tokens against the target's logits (the target's
// standard accept/reject rule under greedy decoding, which the MASW page keeps unchanged; rejected
// speculative draft KV is then discarded, section 4.3 of the same page).
//
// Row i of sequence b (logits [b][i][:], i = 0..k) scores the token that follows the prefix and
// the first i drafts. Kernel 1 splits every row into kAcceptChunk-entry chunks, one workgroup each,
// and leaves the chunk's maximum and the lowest index holding it. Kernel 2 (one wavefront per
// sequence) reduces the chunks of each row in index order (ties keep the lower index), then keeps
// draft i while it equals the choice of row i and every earlier draft was kept: n_accept = the
// kept count a, next_token = the choice at row a, n_drop = k - a (what a ring rollback discards).

#include "wmtp_internal.h"

namespace wmtp {
namespace {

constexpr int kThreads = 256;

// (value, index) with the larger value first, then the lower index
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float to_float(const void* p, size_t i, int dtype) {
  if (dtype == WMTP_BF16) {
    const uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
    return __builtin_bit_cast(float, bits);
  }
  return static_cast<const float*>(p)[i];
}

__global__ __launch_bounds__(kThreads) void argmax_chunk_kernel(AcceptArgs a) {
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;  // b * (k + 1) + i
  const int beg = chunk * kAcceptChunk;
  const int end = min(a.vocab, beg + kAcceptChunk);
  const size_t base = (size_t)row * a.vocab;
  float bv = -INFINITY;
  int bi = 0x7fffffff;  // no entry seen: loses to every real entry, -inf included
  for (int i = beg + threadIdx.x; i < end; i += kThreads) {
    const float v = to_float(a.logits, base + i, a.dtype);
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    a.ws_val[(size_t)row * a.chunks + chunk] = bv;
    a.ws_idx[(size_t)row * a.chunks + chunk] = bi;
  }
}

__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const int k1 = a.k + 1;
  __shared__ int choice[64];
  for (int i = threadIdx.x; i < k1; i += 64) {
    const size_t row = (size_t)b * k1 + i;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < a.chunks; ++c) {
      const float v = a.ws_val[row * a.chunks + c];
      const int x = a.ws_idx[row * a.chunks + c];
      if (better(v, x, bv, bi)) { bv = v; bi = x; }
    }
    choice[i] = bi;
    a.choice[row] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < a.k && a.draft[(size_t)b * a.k + n] == choice[n]) ++n;
    a.n_accept[b] = n;
    a.next_token[b] = choice[n];
    a.n_drop[b] = a.k - n;
  }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  argmax_chunk_kernel<<<dim3(a.chunks, a.batch * (a.k + 1)), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  accept_kernel<<<dim3(a.batch), dim3(64), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace wmtp

// probe.hip -- measurement aids: a streaming read probe, a two-launch hand-off skeleton and a
// last-level-cache flush.
//
// The read probe issues the same 16-byte nontemporal loads as the attention kernels' K/V stream.
// Each of its WMTP_PROBE_BLOCKS workgroups (two per CU) reads one contiguous chunk of the buffer,
// eight loads in flight per thread, and folds what it read into an XOR so that no load can be
// dropped. (Measured on MI355X: contiguous chunks per workgroup reach about 7.1-7.2 TB/s at 512 to
// 2048 workgroups, while a grid-stride walk over the whole buffer falls to about 6 TB/s at 1024
// workgroups and more.) The flush writes a buffer with plain 16-byte stores.

#include <hip/hip_runtime.h>

#include "wmtp.h"
#include "wmtp_probe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4* __restrict__ buf,
                                                              size_t n16, size_t chunk,
                                                              uint32_t* __restrict__ out) {
  const size_t beg = (size_t)blockIdx.x * chunk;
  const size_t end = beg + chunk < n16 ? beg + chunk : n16;
  size_t i = beg + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  // full rounds of kUnroll loads in flight, then the remainder one load at a time
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    u32x4_t x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(buf + i + u * kThreads));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  for (; i < end; i += kThreads)
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(buf + i));
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

// XOR of the 32-bit words of 16-byte words [beg, end) of buf, folded over the workgroup: every
// thread gets the result. 16-byte loads (nontemporal when NT), kUnroll in flight per thread.
template <bool NT>
__device__ uint32_t xor_chunk(const uint4* __restrict__ buf, size_t beg, size_t end) {
  size_t i = beg + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    u32x4_t x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(buf + i + u * kThreads);
      if constexpr (NT) x[u] = __builtin_nontemporal_load(p);
      else x[u] = *p;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  for (; i < end; i += kThreads) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(buf + i);
    if constexpr (NT) acc ^= __builtin_nontemporal_load(p);
    else acc ^= *p;
  }
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < kThreads / 64; ++w) r ^= part[w];
  return r;
}

// launch 1 of the hand-off: read a share of buf, then write this workgroup's partial
__global__ __launch_bounds__(kThreads) void handoff_split_kernel(const uint4* __restrict__ buf,
                                                                 size_t n16, size_t chunk,
                                                                 uint4* __restrict__ parts,
                                                                 size_t part16) {
  const size_t beg = min((size_t)blockIdx.x * chunk, n16);
  const size_t end = min(beg + chunk, n16);
  const uint32_t c = xor_chunk<true>(buf, beg, end);
  uint4* mine = parts + (size_t)blockIdx.x * part16;
  for (size_t i = threadIdx.x; i < part16; i += kThreads)
    mine[i] = make_uint4(c + (uint32_t)i, blockIdx.x, (uint32_t)i, 0u);
}

// launch 2: read a share of all partials, one XOR per workgroup
__global__ __launch_bounds__(kThreads) void handoff_merge_kernel(const uint4* __restrict__ parts,
                                                                 size_t n16, size_t chunk,
                                                                 uint32_t* __restrict__ out) {
  const size_t beg = min((size_t)blockIdx.x * chunk, n16);
  const size_t end = min(beg + chunk, n16);
  const uint32_t r = xor_chunk<false>(parts, beg, end);
  if (threadIdx.x == 0) out[blockIdx.x] = r;
}

__global__ __launch_bounds__(kThreads) void llc_flush_kernel(uint4* __restrict__ buf, size_t n16,
                                                             uint32_t word) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  const uint4 w = make_uint4(word, word, word, word);
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) buf[i] = w;
}

bool ok_buffer(const void* p, size_t bytes) {
  return p && (reinterpret_cast<uintptr_t>(p) % 16) == 0 && bytes > 0 && bytes % 16 == 0;
}

}  // namespace

extern "C" {

int wmtp_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!ok_buffer(buf, bytes) || !out || (reinterpret_cast<uintptr_t>(out) % 4) != 0)
    return WMTP_ERR_INVALID_ARG;
  hipLaunchKernelGGL(probe_read_kernel, dim3(WMTP_PROBE_BLOCKS), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     (bytes / 16 + WMTP_PROBE_BLOCKS - 1) / WMTP_PROBE_BLOCKS, out);
  return hipGetLastError() == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

int wmtp_probe_handoff(const void* buf, size_t bytes, int32_t n_groups, void* parts,
                       size_t part_bytes, uint32_t* out, void* stream) {
  if (!ok_buffer(buf, bytes) || n_groups < 1 || n_groups > 65535) return WMTP_ERR_INVALID_ARG;
  if (part_bytes == 0 || part_bytes % 16 != 0 || part_bytes > ((size_t)1 << 40) / (size_t)n_groups ||
      !ok_buffer(parts, part_bytes * (size_t)n_groups))
    return WMTP_ERR_INVALID_ARG;
  if (!out || (reinterpret_cast<uintptr_t>(out) % 4) != 0) return WMTP_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16, part16 = part_bytes / 16, total16 = part16 * (size_t)n_groups;
  hipLaunchKernelGGL(handoff_split_kernel, dim3(n_groups), dim3(kThreads), 0, s,
                     static_cast<const uint4*>(buf), n16, (n16 + n_groups - 1) / n_groups,
                     static_cast<uint4*>(parts), part16);
  if (hipGetLastError() != hipSuccess) return WMTP_ERR_HIP;
  hipLaunchKernelGGL(handoff_merge_kernel, dim3(WMTP_PROBE_HANDOFF_BLOCKS), dim3(kThreads), 0, s,
                     static_cast<const uint4*>(parts), total16,
                     (total16 + WMTP_PROBE_HANDOFF_BLOCKS - 1) / WMTP_PROBE_HANDOFF_BLOCKS, out);
  return hipGetLastError() == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

int wmtp_llc_flush(void* buf, size_t bytes, uint8_t value, void* stream) {
  if (!ok_buffer(buf, bytes)) return WMTP_ERR_INVALID_ARG;
  const uint32_t word = 0x01010101u * value;
  hipLaunchKernelGGL(llc_flush_kernel, dim3(WMTP_PROBE_BLOCKS), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(buf), bytes / 16, word);
  return hipGetLastError() == hipSuccess ? WMTP_OK : WMTP_ERR_HIP;
}

}  // extern "C"

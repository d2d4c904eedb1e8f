/*
 * wmtp_c_caller.c -- a plain C caller of libwmtp.so (include/wmtp.h): device memory comes from the
 * HIP runtime, and there is no torch and no Python on this path. Test infrastructure: the GPU test
 * tests/test_gpu_c_caller.py runs it and compares what it writes with the float64 oracle.
 *
 * It builds a compact ring buffer (the Windowed-MTP abstract's last sentence: S sink slots plus W
 * window slots) and a contiguous cache from the same N tokens, appending all of them with
 * wmtp_ring_append. It then runs one windowed draft read over the ring, which attends the sinks and
 * the last W tokens, and one full-context read over the cache, which attends all N tokens. It also
 * checks two refused calls. Inputs and outputs are written as raw little-endian files into OUTDIR.
 *
 * Inputs: xorshift64* (Vigna, "An experimental exploration of Marsaglia's xorshift generators,
 * scrambled", ACM TOMS 2016) draws, uniform in [-1, 1), truncated to bf16.
 *
 * usage: wmtp_c_caller OUTDIR     exit status 0 on success, 1 on a failed call or check.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "wmtp.h"

enum { HKV = 2, GQ = 4, HQ = HKV * GQ, D = 128, S = 4, W = 64, N = 300 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ull;
}

static uint16_t next_bf16(void) {
  const double u = (double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0;
  const float f = (float)u;
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(bits >> 16);
}

#define HIP_OK(call)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                   \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

#define WMTP_OK_(call)                                                                    \
  do {                                                                                    \
    int s_ = (call);                                                                      \
    if (s_ != WMTP_OK) {                                                                  \
      fprintf(stderr, "%s returned %d (%s)\n", #call, s_, wmtp_status_string(s_));        \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

static int dump(const char* dir, const char* name, const void* host, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    if (f) fclose(f);
    return 1;
  }
  fclose(f);
  return 0;
}

static int fetch_and_dump(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes);
  if (!host) return 1;
  if (hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    free(host);
    return 1;
  }
  const int rc = dump(dir, name, host, bytes);
  free(host);
  return rc;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTDIR\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  const size_t tok_elems = (size_t)N * HKV * D;  /* new tokens, [1][N][HKV][D] */
  const size_t ring_slots = S + W;
  const size_t ring_elems = (size_t)HKV * ring_slots * D;
  const size_t cache_elems = (size_t)HKV * N * D;
  uint16_t* kn = malloc(tok_elems * 2);
  uint16_t* vn = malloc(tok_elems * 2);
  uint16_t* q = malloc((size_t)HQ * D * 2);
  if (!kn || !vn || !q) return 1;
  for (size_t i = 0; i < tok_elems; ++i) kn[i] = next_bf16();
  for (size_t i = 0; i < tok_elems; ++i) vn[i] = next_bf16();
  for (size_t i = 0; i < (size_t)HQ * D; ++i) q[i] = next_bf16();

  void *d_kn, *d_vn, *d_q, *rk, *rv, *ck, *cv, *ws_w, *ws_f;
  int32_t *rpos, *rlen, *clen;
  float *out_w, *lse_w, *out_f, *lse_f;
  const size_t wsb_w = wmtp_attn_workspace_bytes(1, HQ, HKV, D, 1, (int32_t)ring_slots);
  const size_t wsb_f = wmtp_attn_workspace_bytes(1, HQ, HKV, D, 1, N);
  if (wsb_w == 0 || wsb_f == 0) {
    fprintf(stderr, "no workspace size for these shapes\n");
    return 1;
  }
  HIP_OK(hipMalloc(&d_kn, tok_elems * 2));
  HIP_OK(hipMalloc(&d_vn, tok_elems * 2));
  HIP_OK(hipMalloc(&d_q, (size_t)HQ * D * 2));
  HIP_OK(hipMalloc(&rk, ring_elems * 2));
  HIP_OK(hipMalloc(&rv, ring_elems * 2));
  HIP_OK(hipMalloc((void**)&rpos, ring_slots * 4));
  HIP_OK(hipMalloc((void**)&rlen, 4));
  HIP_OK(hipMalloc(&ck, cache_elems * 2));
  HIP_OK(hipMalloc(&cv, cache_elems * 2));
  HIP_OK(hipMalloc((void**)&clen, 4));
  HIP_OK(hipMalloc((void**)&out_w, (size_t)HQ * D * 4));
  HIP_OK(hipMalloc((void**)&lse_w, (size_t)HQ * 4));
  HIP_OK(hipMalloc((void**)&out_f, (size_t)HQ * D * 4));
  HIP_OK(hipMalloc((void**)&lse_f, (size_t)HQ * 4));
  HIP_OK(hipMalloc(&ws_w, wsb_w));  /* hipMalloc returns 256-byte aligned memory */
  HIP_OK(hipMalloc(&ws_f, wsb_f));
  HIP_OK(hipMemcpy(d_kn, kn, tok_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_vn, vn, tok_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_q, q, (size_t)HQ * D * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(rk, 0, ring_elems * 2));
  HIP_OK(hipMemset(rv, 0, ring_elems * 2));
  HIP_OK(hipMemset(rpos, 0xFF, ring_slots * 4));  /* every tag -1: no position yet */
  HIP_OK(hipMemset(rlen, 0, 4));
  HIP_OK(hipMemset(clen, 0, 4));

  wmtp_kv ring = {rk, rv, rpos, rlen, 1, HKV, D, (int32_t)ring_slots, S, W, WMTP_BF16};
  wmtp_kv cache = {ck, cv, NULL, clen, 1, HKV, D, N, N, 0, WMTP_BF16};
  const float scale = 1.0f / sqrtf((float)D);

  WMTP_OK_(wmtp_ring_append(&ring, d_kn, d_vn, N, NULL));
  WMTP_OK_(wmtp_ring_append(&cache, d_kn, d_vn, N, NULL));
  WMTP_OK_(wmtp_draft_attn_windowed(&ring, d_q, HQ, scale, out_w, lse_w, ws_w, wsb_w, NULL));
  WMTP_OK_(wmtp_draft_attn_full(&cache, d_q, HQ, scale, N, out_f, lse_f, ws_f, wsb_f, NULL));

  /* refused before anything is launched: half the workspace, and a windowed read of a cache that
   * is not a ring */
  if (wmtp_draft_attn_windowed(&ring, d_q, HQ, scale, out_w, lse_w, ws_w, wsb_w / 2, NULL) !=
      WMTP_ERR_WORKSPACE) {
    fprintf(stderr, "an undersized workspace was accepted\n");
    return 1;
  }
  if (wmtp_draft_attn_windowed(&cache, d_q, HQ, scale, out_w, lse_w, ws_w, wsb_w, NULL) !=
      WMTP_ERR_INVALID_ARG) {
    fprintf(stderr, "a contiguous cache was accepted by the windowed read\n");
    return 1;
  }
  if (!wmtp_status_string(WMTP_ERR_WORKSPACE)) return 1;
  HIP_OK(hipDeviceSynchronize());

  if (dump(dir, "k_new.bin", kn, tok_elems * 2) || dump(dir, "v_new.bin", vn, tok_elems * 2) ||
      dump(dir, "q.bin", q, (size_t)HQ * D * 2) ||
      fetch_and_dump(dir, "out_windowed.bin", out_w, (size_t)HQ * D * 4) ||
      fetch_and_dump(dir, "lse_windowed.bin", lse_w, (size_t)HQ * 4) ||
      fetch_and_dump(dir, "out_full.bin", out_f, (size_t)HQ * D * 4) ||
      fetch_and_dump(dir, "lse_full.bin", lse_f, (size_t)HQ * 4) ||
      fetch_and_dump(dir, "ring_k.bin", rk, ring_elems * 2) ||
      fetch_and_dump(dir, "ring_v.bin", rv, ring_elems * 2) ||
      fetch_and_dump(dir, "ring_pos.bin", rpos, ring_slots * 4) ||
      fetch_and_dump(dir, "ring_len.bin", rlen, 4) || fetch_and_dump(dir, "cache_len.bin", clen, 4))
    return 1;
  printf("wmtp_c_caller: ok\n");
  return 0;
}

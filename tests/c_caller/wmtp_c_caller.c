/*
 * wmtp_c_caller.c -- a plain C caller of libwmtp.so (include/wmtp.h): device memory comes from the
 * HIP runtime, and there is no torch and no Python on this path. Test infrastructure: the GPU test
 * tests/test_gpu_c_caller.py runs it and compares what it writes with the float64 oracle.
 *
 * It builds a compact ring buffer (the Windowed-MTP abstract's last sentence: S sink slots plus W
 * window slots) and a contiguous cache from the same N tokens, appending all of them with
 * wmtp_ring_append. It then runs one windowed draft read over the ring, which attends the sinks and
 * the last W tokens, and one full-context read over the cache, which attends all N tokens. A third
 * cache, contiguous, takes the same N tokens and then the target's verification of MV candidates
 * (wmtp_verify_step: append MV candidate tokens and attend them causally, MV * GQ = 32 query rows
 * per KV head) and a second verification of the last MV3 positions (wmtp_verify_attn, MV3 * GQ =
 * 12 rows). A fourth cache, a ring with SLACK extra window slots, takes the same N tokens and then
 * one speculative iteration: an allocation-free draft step (wmtp_draft_step_windowed_noalloc)
 * appends and attends one draft token, wmtp_greedy_accept checks K_ACC draft tokens against
 * float32 logits (the first draft is the argmax of row 0, so it is accepted unless row 0 ties),
 * and wmtp_ring_rollback discards as many tokens as the device-computed n_drop says. Finally a
 * MASW-style read (wmtp_draft_attn_masw) attends the compact ring plus NSLOT memory-slot rows held
 * in a fifth, contiguous cache. It also checks three refused calls. Inputs and outputs are written
 * as raw little-endian files into OUTDIR.
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

enum { HKV = 2, GQ = 4, HQ = HKV * GQ, D = 128, S = 4, W = 64, N = 300, MV = 8, MV3 = 3 };
enum { NV = N + MV, NV_CAP = NV + 5 };  /* verification cache: length after the step, capacity */
enum { SLACK = 4, K_ACC = 2, VOCAB = 1000, NSLOT = 37, SLOT_CAP = 40 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ull;
}

static float next_f32(void) {
  return (float)((double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static uint16_t next_bf16(void) {
  const float f = next_f32();
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
  const size_t cand_elems = (size_t)MV * HKV * D;  /* candidates, [1][MV][HKV][D] */
  const size_t qv_elems = (size_t)MV * HQ * D, qv3_elems = (size_t)MV3 * HQ * D;
  uint16_t* kc = malloc(cand_elems * 2);
  uint16_t* vcn = malloc(cand_elems * 2);
  uint16_t* qv = malloc(qv_elems * 2);
  uint16_t* qv3 = malloc(qv3_elems * 2);
  if (!kc || !vcn || !qv || !qv3) return 1;
  for (size_t i = 0; i < cand_elems; ++i) kc[i] = next_bf16();
  for (size_t i = 0; i < cand_elems; ++i) vcn[i] = next_bf16();
  for (size_t i = 0; i < qv_elems; ++i) qv[i] = next_bf16();
  for (size_t i = 0; i < qv3_elems; ++i) qv3[i] = next_bf16();
  /* the speculative iteration: one draft token and its query, the target's logits (row i scores
   * the token after the first i drafts), the drafts; then the memory-slot rows */
  const size_t tok1 = (size_t)HKV * D, slot_elems = (size_t)NSLOT * HKV * D;
  uint16_t* kd = malloc(tok1 * 2);
  uint16_t* vd = malloc(tok1 * 2);
  uint16_t* qd = malloc((size_t)HQ * D * 2);
  float* logits = malloc((size_t)(K_ACC + 1) * VOCAB * 4);
  uint16_t* sk = malloc(slot_elems * 2);
  uint16_t* sv = malloc(slot_elems * 2);
  int32_t drafts[K_ACC];
  if (!kd || !vd || !qd || !logits || !sk || !sv) return 1;
  for (size_t i = 0; i < tok1; ++i) kd[i] = next_bf16();
  for (size_t i = 0; i < tok1; ++i) vd[i] = next_bf16();
  for (size_t i = 0; i < (size_t)HQ * D; ++i) qd[i] = next_bf16();
  for (size_t i = 0; i < (size_t)(K_ACC + 1) * VOCAB; ++i) logits[i] = next_f32();
  for (size_t i = 0; i < slot_elems; ++i) sk[i] = next_bf16();
  for (size_t i = 0; i < slot_elems; ++i) sv[i] = next_bf16();
  {
    int best = 0; /* draft 0: the first maximum of row 0; draft 1: any token but row 1's maximum */
    for (int t = 1; t < VOCAB; ++t)
      if (logits[t] > logits[best]) best = t;
    int best1 = 0;
    for (int t = 1; t < VOCAB; ++t)
      if (logits[VOCAB + t] > logits[VOCAB + best1]) best1 = t;
    drafts[0] = best;
    drafts[1] = (best1 + 1) % VOCAB;
  }

  void *d_kn, *d_vn, *d_q, *rk, *rv, *ck, *cv, *ws_w, *ws_f;
  int32_t *rpos, *rlen, *clen;
  float *out_w, *lse_w, *out_f, *lse_f;
  const size_t wsb_w = wmtp_attn_workspace_bytes(1, HQ, HKV, D, 1, (int32_t)ring_slots);
  const size_t wsb_f = wmtp_attn_workspace_bytes(1, HQ, HKV, D, 1, N);
  const size_t wsb_v = wmtp_attn_workspace_bytes(1, HQ, HKV, D, MV, NV);
  const size_t wsb_v3 = wmtp_attn_workspace_bytes(1, HQ, HKV, D, MV3, NV);
  const size_t vc_elems = (size_t)HKV * NV_CAP * D;
  void *d_kc, *d_vcn, *d_qv, *d_qv3, *vk, *vv, *ws_v, *ws_v3;
  int32_t* vlen;
  float *out_v, *lse_v, *out_v3, *lse_v3;
  if (wsb_w == 0 || wsb_f == 0 || wsb_v == 0 || wsb_v3 == 0) {
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
  HIP_OK(hipMalloc(&d_kc, cand_elems * 2));
  HIP_OK(hipMalloc(&d_vcn, cand_elems * 2));
  HIP_OK(hipMalloc(&d_qv, qv_elems * 2));
  HIP_OK(hipMalloc(&d_qv3, qv3_elems * 2));
  HIP_OK(hipMalloc(&vk, vc_elems * 2));
  HIP_OK(hipMalloc(&vv, vc_elems * 2));
  HIP_OK(hipMalloc((void**)&vlen, 4));
  HIP_OK(hipMalloc((void**)&out_v, qv_elems * 4));  /* float32 [1][MV][HQ][D] */
  HIP_OK(hipMalloc((void**)&lse_v, (size_t)MV * HQ * 4));
  HIP_OK(hipMalloc((void**)&out_v3, qv3_elems * 4));
  HIP_OK(hipMalloc((void**)&lse_v3, (size_t)MV3 * HQ * 4));
  HIP_OK(hipMalloc(&ws_v, wsb_v));
  HIP_OK(hipMalloc(&ws_v3, wsb_v3));
  HIP_OK(hipMemcpy(d_kc, kc, cand_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_vcn, vcn, cand_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_qv, qv, qv_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_qv3, qv3, qv3_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(vlen, 0, 4));

  const int32_t ring2_slots = S + W + SLACK;
  const size_t ring2_elems = (size_t)HKV * ring2_slots * D;
  const size_t wsb_acc = wmtp_accept_workspace_bytes(1, K_ACC, VOCAB);
  const size_t wsb_m = wmtp_masw_workspace_bytes(1, HQ, HKV, D, (int32_t)ring_slots, NSLOT);
  if (wsb_acc == 0 || wsb_m == 0) {
    fprintf(stderr, "no workspace size for the speculative calls\n");
    return 1;
  }
  void *r2k, *r2v, *d_kd, *d_vd, *d_qd, *d_logits, *ws_acc, *slk, *slv, *d_sk, *d_sv, *ws_m;
  int32_t *r2pos, *r2len, *d_drafts, *choice, *n_accept, *next_tok, *n_drop, *slen;
  float *out_s, *lse_s, *out_m, *lse_m;
  HIP_OK(hipMalloc(&r2k, ring2_elems * 2));
  HIP_OK(hipMalloc(&r2v, ring2_elems * 2));
  HIP_OK(hipMalloc((void**)&r2pos, (size_t)ring2_slots * 4));
  HIP_OK(hipMalloc((void**)&r2len, 4));
  HIP_OK(hipMalloc(&d_kd, tok1 * 2));
  HIP_OK(hipMalloc(&d_vd, tok1 * 2));
  HIP_OK(hipMalloc(&d_qd, (size_t)HQ * D * 2));
  HIP_OK(hipMalloc(&d_logits, (size_t)(K_ACC + 1) * VOCAB * 4));
  HIP_OK(hipMalloc(&ws_acc, wsb_acc));
  HIP_OK(hipMalloc((void**)&d_drafts, K_ACC * 4));
  HIP_OK(hipMalloc((void**)&choice, (K_ACC + 1) * 4));
  HIP_OK(hipMalloc((void**)&n_accept, 4));
  HIP_OK(hipMalloc((void**)&next_tok, 4));
  HIP_OK(hipMalloc((void**)&n_drop, 4));
  HIP_OK(hipMalloc((void**)&out_s, (size_t)HQ * D * 4));
  HIP_OK(hipMalloc((void**)&lse_s, (size_t)HQ * 4));
  HIP_OK(hipMalloc(&slk, (size_t)HKV * SLOT_CAP * D * 2));
  HIP_OK(hipMalloc(&slv, (size_t)HKV * SLOT_CAP * D * 2));
  HIP_OK(hipMalloc((void**)&slen, 4));
  HIP_OK(hipMalloc(&d_sk, slot_elems * 2));
  HIP_OK(hipMalloc(&d_sv, slot_elems * 2));
  HIP_OK(hipMalloc(&ws_m, wsb_m));
  HIP_OK(hipMalloc((void**)&out_m, (size_t)HQ * D * 4));
  HIP_OK(hipMalloc((void**)&lse_m, (size_t)HQ * 4));
  HIP_OK(hipMemcpy(d_kd, kd, tok1 * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_vd, vd, tok1 * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_qd, qd, (size_t)HQ * D * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_logits, logits, (size_t)(K_ACC + 1) * VOCAB * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_drafts, drafts, K_ACC * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_sk, sk, slot_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_sv, sv, slot_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(r2k, 0, ring2_elems * 2));
  HIP_OK(hipMemset(r2v, 0, ring2_elems * 2));
  HIP_OK(hipMemset(r2pos, 0xFF, (size_t)ring2_slots * 4));
  HIP_OK(hipMemset(r2len, 0, 4));
  HIP_OK(hipMemset(slen, 0, 4));
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

  /* verification: the prefix, then the MV candidates appended and verified in one call, then the
   * last MV3 positions verified again by the attention-only call */
  wmtp_kv vcache = {vk, vv, NULL, vlen, 1, HKV, D, NV_CAP, NV_CAP, 0, WMTP_BF16};
  WMTP_OK_(wmtp_ring_append(&vcache, d_kn, d_vn, N, NULL));
  WMTP_OK_(wmtp_verify_step(&vcache, d_kc, d_vcn, d_qv, MV, HQ, scale, NV, out_v, lse_v, ws_v,
                            wsb_v, NULL));
  WMTP_OK_(wmtp_verify_attn(&vcache, d_qv3, MV3, HQ, scale, NV, out_v3, lse_v3, ws_v3, wsb_v3,
                            NULL));

  /* one speculative iteration on a ring with slack: an allocation-free draft step (no workspace
   * argument), greedy accept, and the rollback by the device's count of rejected drafts */
  wmtp_kv ring2 = {r2k, r2v, r2pos, r2len, 1, HKV, D, ring2_slots, S, W, WMTP_BF16};
  WMTP_OK_(wmtp_ring_append(&ring2, d_kn, d_vn, N, NULL));
  WMTP_OK_(wmtp_draft_step_windowed_noalloc(&ring2, d_kd, d_vd, d_qd, HQ, scale, out_s, lse_s,
                                            NULL));
  WMTP_OK_(wmtp_greedy_accept(d_logits, WMTP_F32, 1, K_ACC, VOCAB, d_drafts, choice, n_accept,
                              next_tok, n_drop, ws_acc, wsb_acc, NULL));
  WMTP_OK_(wmtp_ring_rollback(&ring2, n_drop, NULL));

  /* MASW-style read: the compact ring's sinks and window plus NSLOT memory slots */
  wmtp_kv slots = {slk, slv, NULL, slen, 1, HKV, D, SLOT_CAP, SLOT_CAP, 0, WMTP_BF16};
  WMTP_OK_(wmtp_ring_append(&slots, d_sk, d_sv, NSLOT, NULL));
  WMTP_OK_(wmtp_draft_attn_masw(&ring, &slots, d_q, HQ, scale, NSLOT, out_m, lse_m, ws_m, wsb_m,
                                NULL));

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
  if (wmtp_verify_attn(&vcache, d_qv, 17, HQ, scale, NV, out_v, lse_v, ws_v, wsb_v, NULL) !=
      WMTP_ERR_INVALID_ARG) {
    fprintf(stderr, "a verification of 17 candidates was accepted\n");
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
      fetch_and_dump(dir, "ring_len.bin", rlen, 4) || fetch_and_dump(dir, "cache_len.bin", clen, 4) ||
      dump(dir, "k_cand.bin", kc, cand_elems * 2) || dump(dir, "v_cand.bin", vcn, cand_elems * 2) ||
      dump(dir, "q_verify.bin", qv, qv_elems * 2) || dump(dir, "q_verify3.bin", qv3, qv3_elems * 2) ||
      fetch_and_dump(dir, "out_verify_step.bin", out_v, qv_elems * 4) ||
      fetch_and_dump(dir, "lse_verify_step.bin", lse_v, (size_t)MV * HQ * 4) ||
      fetch_and_dump(dir, "out_verify.bin", out_v3, qv3_elems * 4) ||
      fetch_and_dump(dir, "lse_verify.bin", lse_v3, (size_t)MV3 * HQ * 4) ||
      fetch_and_dump(dir, "verify_k.bin", vk, vc_elems * 2) ||
      fetch_and_dump(dir, "verify_v.bin", vv, vc_elems * 2) ||
      fetch_and_dump(dir, "verify_len.bin", vlen, 4) ||
      dump(dir, "k_draft.bin", kd, tok1 * 2) || dump(dir, "v_draft.bin", vd, tok1 * 2) ||
      dump(dir, "q_draft.bin", qd, (size_t)HQ * D * 2) ||
      fetch_and_dump(dir, "out_noalloc.bin", out_s, (size_t)HQ * D * 4) ||
      fetch_and_dump(dir, "lse_noalloc.bin", lse_s, (size_t)HQ * 4) ||
      dump(dir, "logits.bin", logits, (size_t)(K_ACC + 1) * VOCAB * 4) ||
      dump(dir, "drafts.bin", drafts, K_ACC * 4) ||
      fetch_and_dump(dir, "choice.bin", choice, (K_ACC + 1) * 4) ||
      fetch_and_dump(dir, "n_accept.bin", n_accept, 4) ||
      fetch_and_dump(dir, "next_token.bin", next_tok, 4) ||
      fetch_and_dump(dir, "n_drop.bin", n_drop, 4) ||
      fetch_and_dump(dir, "ring2_pos.bin", r2pos, (size_t)ring2_slots * 4) ||
      fetch_and_dump(dir, "ring2_len.bin", r2len, 4) ||
      fetch_and_dump(dir, "ring2_k.bin", r2k, ring2_elems * 2) ||
      fetch_and_dump(dir, "ring2_v.bin", r2v, ring2_elems * 2) ||
      dump(dir, "slots_k.bin", sk, slot_elems * 2) || dump(dir, "slots_v.bin", sv, slot_elems * 2) ||
      fetch_and_dump(dir, "out_masw.bin", out_m, (size_t)HQ * D * 4) ||
      fetch_and_dump(dir, "lse_masw.bin", lse_m, (size_t)HQ * 4))
    return 1;
  printf("wmtp_c_caller: ok\n");
  return 0;
}

/*
 * wmtp_oracle.c -- float64 CPU oracle for softmax attention over an explicit set of KV rows.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file; only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark do. It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes (Windowed-MTP abstract, thelatestinai.com/papers/2607.21535, and the same text
 * on the khansong-paper-with-me page): both the native draft head and the windowed draft head run
 * ordinary softmax attention; windowing only changes WHICH cached tokens are attended (attention
 * sinks plus a recent sliding window), and verification stays full attention. So for one query
 * vector q and an attended set A of cached rows (k_p, v_p):
 *
 *     s_p = scale * sum_i q_i k_{p,i}            for p in A
 *     M   = max_{p in A} s_p
 *     Z   = sum_{p in A} exp(s_p - M)
 *     o   = sum_{p in A} exp(s_p - M) v_p / Z
 *     lse = M + ln Z
 *
 * This is the plain definition written out: two passes over A, float64 throughout, no online
 * rescaling, no splitting of A, no blocking. bf16 inputs are widened exactly (a bf16 value is the
 * top 16 bits of a float32). Which rows form A (sinks, window, causal verify prefix) is decided by
 * the Python side of the oracle, which passes each problem's rows as up to ORACLE_RUNS contiguous
 * runs (sinks, the recent window and, for the MASW layout, the memory slots).
 *
 * Degenerate case (a reading; the pages are silent): an empty set gives o = 0 and lse = -inf.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: IEEE semantics and program order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };
#define ORACLE_RUNS 4

/* One attention problem: a query vector and the rows it attends. Row r of run s starts at element
 * kv_off[s] + r * row_stride of the K and V arrays. All offsets are in elements. */
typedef struct {
  int64_t q_off;       /* element offset of the query vector in q */
  int64_t kv_off[ORACLE_RUNS]; /* element offset of the first row of each run */
  int64_t count[ORACLE_RUNS];  /* rows in each run (0 for an unused run) */
  int64_t row_stride;  /* elements between consecutive rows of a run */
  int64_t out_off;     /* element offset of the output vector in out; lse index is out_off / d */
} wmtp_oracle_problem;

static double load_elem(const void* base, int32_t dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  if (dtype == ORACLE_F64) return ((const double*)base)[i];
  /* bf16: the 16 stored bits are the high half of an IEEE float32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static void solve_one(const wmtp_oracle_problem* pr, int32_t d, int32_t dtype_q, int32_t dtype_kv,
                      const void* q, const void* k, const void* v, double scale, double* out,
                      double* lse) {
  int64_t n = 0;
  for (int run = 0; run < ORACLE_RUNS; ++run) n += pr->count[run];
  double* o = out + pr->out_off;
  for (int32_t i = 0; i < d; ++i) o[i] = 0.0;
  if (n <= 0) {
    lse[pr->out_off / d] = -INFINITY;
    return;
  }
  double* qd = (double*)malloc(sizeof(double) * (size_t)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  for (int32_t i = 0; i < d; ++i) qd[i] = load_elem(q, dtype_q, pr->q_off + i);

  /* pass 1: scores and their maximum */
  int64_t j = 0;
  double M = -INFINITY;
  for (int run = 0; run < ORACLE_RUNS; ++run) {
    for (int64_t r = 0; r < pr->count[run]; ++r, ++j) {
      int64_t base = pr->kv_off[run] + r * pr->row_stride;
      double dot = 0.0;
      for (int32_t i = 0; i < d; ++i) dot += qd[i] * load_elem(k, dtype_kv, base + i);
      s[j] = scale * dot;
      if (s[j] > M) M = s[j];
    }
  }
  /* pass 2: normaliser and weighted sum of values */
  double Z = 0.0;
  j = 0;
  for (int run = 0; run < ORACLE_RUNS; ++run) {
    for (int64_t r = 0; r < pr->count[run]; ++r, ++j) {
      int64_t base = pr->kv_off[run] + r * pr->row_stride;
      double w = exp(s[j] - M);
      Z += w;
      for (int32_t i = 0; i < d; ++i) o[i] += w * load_elem(v, dtype_kv, base + i);
    }
  }
  for (int32_t i = 0; i < d; ++i) o[i] /= Z;
  lse[pr->out_off / d] = M + log(Z);
  free(s);
  free(qd);
}

/* Solve nprob independent problems. Returns 0, or 1 on a bad argument. nthreads <= 0 means the
 * OpenMP default. Problems are independent, so they are spread over threads whole; the arithmetic
 * of each problem is sequential and does not depend on the thread count. */
int wmtp_oracle_attention(int64_t nprob, const wmtp_oracle_problem* probs, int32_t d,
                          int32_t dtype_q, int32_t dtype_kv, const void* q, const void* k,
                          const void* v, double scale, double* out, double* lse,
                          int32_t nthreads) {
  if (nprob < 0 || d <= 0 || (nprob > 0 && (!probs || !q || !out || !lse))) return 1;
  for (int64_t p = 0; p < nprob; ++p) {
    int64_t total = 0;
    for (int run = 0; run < ORACLE_RUNS; ++run) {
      if (probs[p].count[run] < 0) return 1;
      total += probs[p].count[run];
    }
    if (total > 0 && (!k || !v)) return 1;
    if (probs[p].out_off % d != 0) return 1;
  }
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
  for (int64_t p = 0; p < nprob; ++p)
    solve_one(&probs[p], d, dtype_q, dtype_kv, q, k, v, scale, out, lse);
  (void)nthreads;
  return 0;
}

/* Number of threads the OpenMP runtime would use by default (reported with CPU timings). */
int wmtp_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

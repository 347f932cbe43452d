/* Host driver for the sanitizer build of oracle/oracle.c (AddressSanitizer and
 * UndefinedBehaviorSanitizer): runs every entry point on tiny inputs, with
 * several threads, all three input types, empty sequences and invalid
 * arguments, and checks closed forms the definition fixes (a single key gives
 * O = V exactly and LSE = scale q.k; an empty decode sequence gives O = 0 and
 * LSE = -inf).  Prints "ORACLE SANITIZE OK" and returns 0 when every check
 * holds; any memory or undefined-behaviour error aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_version(void);
int oracle_attn_rows(int dtype, const void *q, const void *k, const void *v, int B, int Hq, int Hkv, int N, int Nk,
                     int d, int causal, double scale, int64_t nrows, const int32_t *rb, const int32_t *rh,
                     const int32_t *ri, double *o_out, double *lse_out, int nthreads);
int oracle_decode_rows(int dtype, const void *q, const void *k_cache, const void *v_cache, const int32_t *cu, int B,
                       int Hq, int Hkv, int d, double scale, int64_t nrows, const int32_t *rb, const int32_t *rh,
                       double *o_out, double *lse_out, int nthreads);

static uint32_t lcg_state = 12345u;
static double urand(void) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return ((lcg_state >> 8) / 16777216.0) * 2.0 - 1.0;
}
static int failures = 0;
#define CHECK(c, msg)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      fprintf(stderr, "check failed: %s\n", msg);       \
      ++failures;                                       \
    }                                                   \
  } while (0)

/* a double rounded to bf16 bits (round to nearest even) and the float bits */
static uint16_t to_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void prefill_case(int dtype, int causal, int N, int Nk, int nthreads) {
  const int B = 2, Hq = 4, Hkv = 2, d = 8;
  const size_t nq = (size_t)B * N * Hq * d, nk = (size_t)B * Nk * Hkv * d;
  const size_t es = dtype == 0 ? 8 : dtype == 1 ? 4 : 2;
  unsigned char *q = malloc(nq * es + 1), *k = malloc(nk * es + 1), *v = malloc(nk * es + 1);
  for (size_t i = 0; i < nq; ++i) {
    const double x = urand();
    if (dtype == 0) ((double *)q)[i] = x; else if (dtype == 1) ((float *)q)[i] = (float)x; else ((uint16_t *)q)[i] = to_bf16(x);
  }
  for (size_t i = 0; i < nk; ++i) {
    const double x = urand(), y = urand();
    if (dtype == 0) { ((double *)k)[i] = x; ((double *)v)[i] = y; }
    else if (dtype == 1) { ((float *)k)[i] = (float)x; ((float *)v)[i] = (float)y; }
    else { ((uint16_t *)k)[i] = to_bf16(x); ((uint16_t *)v)[i] = to_bf16(y); }
  }
  const int64_t nrows = (int64_t)B * Hq * N;
  int32_t *rb = malloc(sizeof(int32_t) * (nrows + 1)), *rh = malloc(sizeof(int32_t) * (nrows + 1)),
          *ri = malloc(sizeof(int32_t) * (nrows + 1));
  int64_t r = 0;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int i = 0; i < N; ++i, ++r) { rb[r] = b; rh[r] = h; ri[r] = i; }
  double *o = malloc(sizeof(double) * (nrows * d + 1)), *lse = malloc(sizeof(double) * (nrows + 1));
  const int rc = oracle_attn_rows(dtype, q, k, v, B, Hq, Hkv, N, Nk, d, causal, 0.7, nrows, rb, rh, ri, o, lse,
                                  nthreads);
  CHECK(rc == 0, "oracle_attn_rows status");
  for (int64_t x = 0; x < nrows * d; ++x) CHECK(!isnan(o[x]), "O is a number");
  if (Nk == 1 && !causal) {
    /* single key: O = V[0] exactly, LSE = scale q.k */
    for (r = 0; r < nrows; ++r)
      for (int c = 0; c < d; ++c) {
        const size_t vi = ((size_t)rb[r] * Nk * Hkv + rh[r] / (Hq / Hkv)) * d + c;
        const double vv = dtype == 0 ? ((double *)v)[vi] : dtype == 1 ? ((float *)v)[vi] : 0.0;
        if (dtype != 2) CHECK(o[r * d + c] == vv, "single key O = V");
      }
  }
  free(q); free(k); free(v); free(rb); free(rh); free(ri); free(o); free(lse);
}

static void decode_case(int nthreads) {
  const int B = 4, Hq = 4, Hkv = 2, d = 8;
  const int32_t cu[5] = {0, 3, 3, 10, 11};   /* sequence 1 is empty */
  const int total = cu[B];
  double *q = malloc(sizeof(double) * B * Hq * d), *kc = malloc(sizeof(double) * total * Hkv * d),
         *vc = malloc(sizeof(double) * total * Hkv * d);
  for (int i = 0; i < B * Hq * d; ++i) q[i] = urand();
  for (int i = 0; i < total * Hkv * d; ++i) { kc[i] = urand(); vc[i] = urand(); }
  const int64_t nrows = (int64_t)B * Hq;
  int32_t rb[16], rh[16];
  for (int b = 0; b < B; ++b) for (int h = 0; h < Hq; ++h) { rb[b * Hq + h] = b; rh[b * Hq + h] = h; }
  double o[16 * 8], lse[16];
  const int rc = oracle_decode_rows(0, q, kc, vc, cu, B, Hq, Hkv, d, 0.5, nrows, rb, rh, o, lse, nthreads);
  CHECK(rc == 0, "oracle_decode_rows status");
  for (int h = 0; h < Hq; ++h) {
    CHECK(isinf(lse[1 * Hq + h]) && lse[1 * Hq + h] < 0, "empty sequence LSE = -inf");
    for (int c = 0; c < d; ++c) CHECK(o[(1 * Hq + h) * d + c] == 0.0, "empty sequence O = 0");
    /* sequence 3 holds one key: O = V exactly */
    for (int c = 0; c < d; ++c) CHECK(o[(3 * Hq + h) * d + c] == vc[((size_t)10 * Hkv + h / 2) * d + c], "single cached key O = V");
  }
  free(q); free(kc); free(vc);
}

int main(void) {
  CHECK(oracle_version() >= 1, "version");
  for (int dtype = 0; dtype < 3; ++dtype)
    for (int causal = 0; causal < 2; ++causal) {
      prefill_case(dtype, causal, 5, 7, 3);
      prefill_case(dtype, causal, 7, 5, 2);   /* N > Nk: leading causal rows see no key */
      prefill_case(dtype, causal, 3, 1, 1);
    }
  decode_case(1);
  decode_case(4);
  /* invalid arguments are refused without touching the buffers */
  int32_t one = 0;
  double sink[8];
  CHECK(oracle_attn_rows(7, sink, sink, sink, 1, 1, 1, 1, 1, 1, 0, 1.0, 1, &one, &one, &one, sink, sink, 1) == 1,
        "bad dtype refused");
  CHECK(oracle_attn_rows(0, sink, sink, sink, 1, 3, 2, 1, 1, 1, 0, 1.0, 1, &one, &one, &one, sink, sink, 1) == 1,
        "Hq not a multiple of Hkv refused");
  int32_t bad = 5;
  CHECK(oracle_attn_rows(0, sink, sink, sink, 1, 1, 1, 1, 1, 1, 0, 1.0, 1, &one, &one, &bad, sink, sink, 1) == 1,
        "row index past N refused");
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ORACLE SANITIZE OK\n");
  return 0;
}

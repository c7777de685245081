/*
 * Drives every entry point of the fp64 oracle (oracle/attn_oracle.c) on small
 * shapes, for the build with -fsanitize=address,undefined that the CPU test
 * suite runs: out-of-bounds accesses, use of freed memory, signed overflow
 * and the like abort the run. It also checks a few facts that hold exactly
 * or to rounding (row 0 of O is V's row 0; the columns of dK sum to zero and
 * those of dV to the sum of dO; the decode of the last row equals that row of
 * the forward; dropout that keeps everything equals no dropout; each row of
 * dS sums to zero) and the status codes of bad arguments. Exit status 0 when
 * everything holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_fwd(long heads, long T, long D, const double* q, const double* k,
                    const double* v, double* o, double* lse, int nthreads);
int oracle_attn_bwd(long heads, long T, long D, const double* q, const double* k,
                    const double* v, const double* dout, double* dq, double* dk, double* dv,
                    int nthreads);
int oracle_attn_head_intermediates(long T, long D, const double* q, const double* k,
                                   const double* v, const double* dout, double* P, double* dP,
                                   double* dS, double* delta);
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
long oracle_dropout_threshold(double p);
int oracle_dropout_keep(long n, const long* bh, long T, double p, uint64_t seed,
                        uint32_t offset, uint8_t* keep);
int oracle_attn_fwd_dropout(long heads, long T, long D, const double* q, const double* k,
                            const double* v, const uint8_t* keep, double z, double* o,
                            double* lse, int nthreads);
int oracle_attn_bwd_dropout(long heads, long T, long D, const double* q, const double* k,
                            const double* v, const double* dout, const uint8_t* keep, double z,
                            double* dq, double* dk, double* dv, int nthreads);
int oracle_attn_decode(long heads, long L, long D, const double* q, const double* k,
                       const double* v, const long* lengths, double* o, double* lse);

static int failures = 0;

static void check(int ok, const char* what, long T, long D) {
  if (!ok) {
    fprintf(stderr, "FAIL %s (T=%ld D=%ld)\n", what, T, D);
    ++failures;
  }
}

static uint64_t lcg = 88172645463325252ull;

static double uniform(void) {  /* in [-1, 1) */
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg >> 11) / 4503599627370496.0 - 1.0;
}

static double* fill(long n) {
  double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) a[i] = 2.0 * uniform();
  return a;
}

static void one_shape(long heads, long T, long D, int threads) {
  const long E = heads * T * D, R = heads * T;
  double *q = fill(E), *k = fill(E), *v = fill(E), *dout = fill(E);
  double *o = fill(E), *lse = fill(R), *dq = fill(E), *dk = fill(E), *dv = fill(E);
  check(oracle_attn_fwd(heads, T, D, q, k, v, o, lse, threads) == 0, "fwd status", T, D);
  check(oracle_attn_bwd(heads, T, D, q, k, v, dout, dq, dk, dv, threads) == 0, "bwd status", T,
        D);
  for (long h = 0; h < heads; ++h) {
    const long b = h * T * D;
    for (long d = 0; d < D; ++d) check(o[b + d] == v[b + d], "row 0 of O is V[0]", T, D);
    for (long d = 0; d < D; ++d) {
      double sk = 0, sv = 0, so = 0, mag = 1e-300;
      for (long t = 0; t < T; ++t) {
        sk += dk[b + t * D + d];
        sv += dv[b + t * D + d];
        so += dout[b + t * D + d];
        mag += fabs(dk[b + t * D + d]) + fabs(dv[b + t * D + d]);
      }
      check(fabs(sk) <= 1e-12 * mag, "sum of dK columns is 0", T, D);
      check(fabs(sv - so) <= 1e-12 * (mag + fabs(so)), "sum of dV is sum of dO", T, D);
    }
  }
  /* Decode of the last row of every head against the forward. */
  double *qd = (double*)malloc(sizeof(double) * (size_t)(heads * D));
  double *od = fill(heads * D), *ld = fill(heads);
  long* len = (long*)malloc(sizeof(long) * (size_t)heads);
  for (long h = 0; h < heads; ++h) {
    memcpy(qd + h * D, q + h * T * D + (T - 1) * D, sizeof(double) * (size_t)D);
    len[h] = T;
  }
  check(oracle_attn_decode(heads, T, D, qd, k, v, len, od, ld) == 0, "decode status", T, D);
  for (long h = 0; h < heads; ++h) {
    for (long d = 0; d < D; ++d)
      check(fabs(od[h * D + d] - o[h * T * D + (T - 1) * D + d]) <= 1e-12, "decode = last row",
            T, D);
    check(fabs(ld[h] - lse[h * T + T - 1]) <= 1e-12, "decode LSE", T, D);
  }
  /* Dropout that keeps everything (p = 0) is the plain attention. */
  long* bh = (long*)malloc(sizeof(long) * (size_t)heads);
  for (long h = 0; h < heads; ++h) bh[h] = h;
  uint8_t* keep = (uint8_t*)malloc((size_t)(heads * T * T));
  check(oracle_dropout_keep(heads, bh, T, 0.0, 7, 1, keep) == 0, "keep status", T, D);
  double *o2 = fill(E), *l2 = fill(R), *dq2 = fill(E), *dk2 = fill(E), *dv2 = fill(E);
  check(oracle_attn_fwd_dropout(heads, T, D, q, k, v, keep, 1.0, o2, l2, threads) == 0,
        "fwd dropout status", T, D);
  check(oracle_attn_bwd_dropout(heads, T, D, q, k, v, dout, keep, 1.0, dq2, dk2, dv2,
                                threads) == 0, "bwd dropout status", T, D);
  for (long i = 0; i < E; ++i) {
    check(fabs(o2[i] - o[i]) <= 1e-12 && fabs(dq2[i] - dq[i]) <= 1e-12 &&
          fabs(dk2[i] - dk[i]) <= 1e-12 && fabs(dv2[i] - dv[i]) <= 1e-12,
          "p = 0 equals no dropout", T, D);
    if (failures) break;
  }
  /* A real mask at p = 0.3 runs too. */
  check(oracle_dropout_keep(heads, bh, T, 0.3, 0xFFFFFFFFFFFFull, 0xFFFFFFFFu, keep) == 0,
        "keep p=0.3", T, D);
  check(oracle_attn_bwd_dropout(heads, T, D, q, k, v, dout, keep, 1.0 / 0.7, dq2, dk2, dv2,
                                threads) == 0, "bwd dropout p=0.3", T, D);
  /* Row sums of dS on head 0. */
  double *P = fill(T * T), *dP = fill(T * T), *dS = fill(T * T), *delta = fill(T);
  check(oracle_attn_head_intermediates(T, D, q, k, v, dout, P, dP, dS, delta) == 0,
        "intermediates status", T, D);
  for (long i = 0; i < T; ++i) {
    double s = 0, mag = 1e-300;
    for (long j = 0; j <= i; ++j) {
      s += dS[i * T + j];
      mag += fabs(P[i * T + j] * dP[i * T + j]);
    }
    check(fabs(s) <= 1e-12 * mag, "row of dS sums to 0", T, D);
  }
  double* bufs[] = {q, k, v, dout, o, lse, dq, dk, dv, qd, od, ld, o2, l2, dq2, dk2, dv2, P, dP,
                    dS, delta};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) free(bufs[i]);
  free(len);
  free(bh);
  free(keep);
}

int main(void) {
  const long Ts[] = {1, 2, 5, 17, 40};
  const long Ds[] = {1, 3, 8, 64};
  for (size_t i = 0; i < sizeof Ts / sizeof Ts[0]; ++i)
    for (size_t j = 0; j < sizeof Ds / sizeof Ds[0]; ++j)
      one_shape(3, Ts[i], Ds[j], (int)(1 + (i + j) % 3));
  /* Bad arguments: status codes, no memory touched. */
  double x = 0;
  uint8_t m = 0;
  long one = 1;
  check(oracle_attn_fwd(-1, 4, 4, &x, &x, &x, &x, &x, 1) != 0, "fwd heads < 0", 4, 4);
  check(oracle_attn_fwd(1, 4, 0, &x, &x, &x, &x, &x, 1) != 0, "fwd D = 0", 4, 0);
  check(oracle_attn_fwd(1, 4, 4, NULL, &x, &x, &x, &x, 1) != 0, "fwd NULL q", 4, 4);
  check(oracle_attn_fwd(0, 4, 4, &x, &x, &x, &x, &x, 1) == 0, "fwd empty", 4, 4);
  check(oracle_attn_bwd(1, 4, 4, &x, &x, &x, &x, NULL, &x, &x, 1) != 0, "bwd NULL dq", 4, 4);
  check(oracle_dropout_threshold(1.0) < 0 && oracle_dropout_threshold(-0.5) < 0 &&
        oracle_dropout_threshold(NAN) < 0, "bad dropout rates", 0, 0);
  check(oracle_dropout_keep(1, &one, 4, 1.5, 0, 0, &m) != 0, "keep bad p", 4, 0);
  check(oracle_attn_decode(1, 4, 4, NULL, &x, &x, &one, &x, &x) != 0, "decode NULL q", 4, 4);
  uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4];
  oracle_philox4x32_10(ctr, key, out);
  /* Philox4x32-10 of the zero counter and key (Salmon et al., SC'11 known-answer). */
  check(out[0] == 0x6627e8d5u && out[1] == 0xe169c58du && out[2] == 0xbc57ac4cu &&
        out[3] == 0x9b00dbd8u, "Philox known answer", 0, 0);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle self-check ok\n");
  return 0;
}

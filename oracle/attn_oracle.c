/*
 * Plain fp64 CPU oracle for causal multi-head self-attention, forward and
 * backward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or constant with the GPU
 * library.
 *
 * What it computes (layout [B, H, T, D], contiguous, row-major):
 *
 *   Forward, the "slow, written-out" attention that nanoGPT's model.py keeps
 *   beside its fused call (page "nanoGPT: a real GPT in two 300-line files",
 *   section 2 "How the code works"): scores q.k^T multiplied by
 *   1/sqrt(head size), every future position set to -infinity, a softmax
 *   over each row, then the product with v. "Causal" means a position sees
 *   only itself and earlier positions (same page, section 8 "Self-check"),
 *   so key j is visible to query i iff j <= i.
 *
 *   For one head, with s = 1/sqrt(D) and j <= i:
 *     S_ij   = s * sum_d Q_id K_jd
 *     m_i    = max_j S_ij,   l_i = sum_j exp(S_ij - m_i)
 *     P_ij   = exp(S_ij - m_i) / l_i          (P_ij = 0 for j > i)
 *     O_i    = sum_j P_ij V_j
 *     LSE_i  = m_i + ln l_i                    (natural log, scaled scores)
 *
 *   Backward: the analytic gradient of L = sum(dO * O) that autograd forms
 *   for nanoGPT's loss.backward() (same page, section 1 "Summary"):
 *     delta_i = sum_d dO_id O_id
 *     dP_ij   = sum_d dO_id V_jd
 *     dS_ij   = P_ij (dP_ij - delta_i)
 *     dV_j    = sum_{i>=j} P_ij dO_i
 *     dQ_i    = s sum_{j<=i} dS_ij K_j
 *     dK_j    = s sum_{i>=j} dS_ij Q_i
 *
 * It is the plain two-pass (max, then sum) softmax per row, not an online
 * one; rows of P are recomputed in the backward instead of being stored.
 * Sums run in ascending index order; exp and log are libm's. Each (b, h) head
 * is computed by exactly one thread, so results do not depend on the thread
 * count.
 *
 * Parity pins (checked by the CPU test suite, independent of this file):
 * 50-digit brute force with the explicit softmax Jacobian, central finite
 * differences, the library routine scaled_dot_product_attention in fp64,
 * closed forms (row 0, all keys equal, T = 1), zero row sums of dS, column
 * sums of dK and dV, and equivariances.
 *
 * Attention dropout (the dropout_p argument of the fused call, same page,
 * section 2) is the second half of this file: a keep mask M drawn from the
 * counter-based generator Philox4x32-10, and forward / backward that take M
 * explicitly (see the block comment there).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* ---- one head ---------------------------------------------------------- */

/* Row i of the attention matrix: fills p[0..i] with P_ij, returns LSE_i. */
static double softmax_row(long i, long D, double s, const double* q,
                          const double* k, double* p) {
  const double* qi = q + i * D;
  double m = -INFINITY;
  for (long j = 0; j <= i; ++j) {
    const double* kj = k + j * D;
    double dot = 0.0;
    for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];
    p[j] = s * dot;
    if (p[j] > m) m = p[j];
  }
  double l = 0.0;
  for (long j = 0; j <= i; ++j) {
    p[j] = exp(p[j] - m);
    l += p[j];
  }
  for (long j = 0; j <= i; ++j) p[j] /= l;
  return m + log(l);
}

static void head_forward(long T, long D, const double* q, const double* k,
                         const double* v, double* o, double* lse, double* p) {
  const double s = 1.0 / sqrt((double)D);
  for (long i = 0; i < T; ++i) {
    double li = softmax_row(i, D, s, q, k, p);
    if (lse) lse[i] = li;
    double* oi = o + i * D;
    for (long d = 0; d < D; ++d) oi[d] = 0.0;
    for (long j = 0; j <= i; ++j) {
      const double* vj = v + j * D;
      for (long d = 0; d < D; ++d) oi[d] += p[j] * vj[d];
    }
  }
}

/* o is scratch of T*D doubles, p of T doubles. */
static void head_backward(long T, long D, const double* q, const double* k,
                          const double* v, const double* dout, double* dq,
                          double* dk, double* dv, double* o, double* p,
                          double* delta) {
  const double s = 1.0 / sqrt((double)D);
  head_forward(T, D, q, k, v, o, NULL, p);
  for (long i = 0; i < T; ++i) {
    double acc = 0.0;
    for (long d = 0; d < D; ++d) acc += dout[i * D + d] * o[i * D + d];
    delta[i] = acc;
  }
  memset(dq, 0, sizeof(double) * T * D);
  memset(dk, 0, sizeof(double) * T * D);
  memset(dv, 0, sizeof(double) * T * D);
  for (long i = 0; i < T; ++i) {
    softmax_row(i, D, s, q, k, p);
    const double* qi = q + i * D;
    const double* doi = dout + i * D;
    double* dqi = dq + i * D;
    for (long j = 0; j <= i; ++j) {
      const double* kj = k + j * D;
      const double* vj = v + j * D;
      double dp = 0.0;
      for (long d = 0; d < D; ++d) dp += doi[d] * vj[d];
      const double ds = p[j] * (dp - delta[i]);
      double* dvj = dv + j * D;
      double* dkj = dk + j * D;
      for (long d = 0; d < D; ++d) {
        dvj[d] += p[j] * doi[d];
        dqi[d] += s * ds * kj[d];
        dkj[d] += s * ds * qi[d];
      }
    }
  }
}

/* ---- threads over heads ------------------------------------------------ */

typedef struct {
  int backward;
  long heads, T, D;
  const double *q, *k, *v, *dout;
  double *o, *lse, *dq, *dk, *dv;
  int tid, nthreads;
  int status;
} job_t;

static void* run_job(void* arg) {
  job_t* jb = (job_t*)arg;
  const long T = jb->T, D = jb->D, E = T * D;
  double* p = (double*)malloc(sizeof(double) * (size_t)T);
  double* o = jb->backward ? (double*)malloc(sizeof(double) * (size_t)E) : NULL;
  double* delta = jb->backward ? (double*)malloc(sizeof(double) * (size_t)T) : NULL;
  if (!p || (jb->backward && (!o || !delta))) {
    jb->status = ORACLE_ENOMEM;
  } else {
    for (long h = jb->tid; h < jb->heads; h += jb->nthreads) {
      if (jb->backward)
        head_backward(T, D, jb->q + h * E, jb->k + h * E, jb->v + h * E,
                      jb->dout + h * E, jb->dq + h * E, jb->dk + h * E,
                      jb->dv + h * E, o, p, delta);
      else
        head_forward(T, D, jb->q + h * E, jb->k + h * E, jb->v + h * E,
                     jb->o + h * E, jb->lse ? jb->lse + h * T : NULL, p);
    }
    jb->status = ORACLE_OK;
  }
  free(p);
  free(o);
  free(delta);
  return NULL;
}

static int run_all(job_t proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 1024) nthreads = 1024;
  if ((long)nthreads > proto.heads) nthreads = (int)(proto.heads > 0 ? proto.heads : 1);
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return ORACLE_ENOMEM;
  }
  int status = ORACLE_OK;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].tid = t;
    jobs[t].nthreads = nthreads;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) break;
    started = t;
  }
  /* Threads that failed to start are run on this thread. */
  run_job(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; ++t) run_job(&jobs[t]);
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != ORACLE_OK) status = jobs[t].status;
  free(jobs);
  free(th);
  return status;
}

/* ---- exported ---------------------------------------------------------- */

/* O [heads, T, D] and LSE [heads, T] (lse may be NULL). heads = B*H. */
int oracle_attn_fwd(long heads, long T, long D, const double* q, const double* k,
                    const double* v, double* o, double* lse, int nthreads) {
  if (heads < 0 || T < 0 || D < 1 || !q || !k || !v || !o) return ORACLE_EINVAL;
  if (heads == 0 || T == 0) return ORACLE_OK;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.backward = 0;
  jb.heads = heads;
  jb.T = T;
  jb.D = D;
  jb.q = q;
  jb.k = k;
  jb.v = v;
  jb.o = o;
  jb.lse = lse;
  return run_all(jb, nthreads);
}

/* dQ, dK, dV [heads, T, D] for the upstream gradient dout [heads, T, D]. */
int oracle_attn_bwd(long heads, long T, long D, const double* q, const double* k,
                    const double* v, const double* dout, double* dq, double* dk,
                    double* dv, int nthreads) {
  if (heads < 0 || T < 0 || D < 1 || !q || !k || !v || !dout || !dq || !dk || !dv)
    return ORACLE_EINVAL;
  if (heads == 0 || T == 0) return ORACLE_OK;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.backward = 1;
  jb.heads = heads;
  jb.T = T;
  jb.D = D;
  jb.q = q;
  jb.k = k;
  jb.v = v;
  jb.dout = dout;
  jb.dq = dq;
  jb.dk = dk;
  jb.dv = dv;
  return run_all(jb, nthreads);
}

/*
 * One head's full T x T intermediates, for small T: P, dP, dS (row-major,
 * zero above the diagonal) and delta [T]. Used by tests of row identities.
 */
int oracle_attn_head_intermediates(long T, long D, const double* q, const double* k,
                                   const double* v, const double* dout, double* P,
                                   double* dP, double* dS, double* delta) {
  if (T < 1 || D < 1 || !q || !k || !v || !dout || !P || !dP || !dS || !delta)
    return ORACLE_EINVAL;
  const double s = 1.0 / sqrt((double)D);
  double* o = (double*)malloc(sizeof(double) * (size_t)(T * D));
  double* p = (double*)malloc(sizeof(double) * (size_t)T);
  if (!o || !p) {
    free(o);
    free(p);
    return ORACLE_ENOMEM;
  }
  head_forward(T, D, q, k, v, o, NULL, p);
  for (long i = 0; i < T; ++i) {
    double acc = 0.0;
    for (long d = 0; d < D; ++d) acc += dout[i * D + d] * o[i * D + d];
    delta[i] = acc;
  }
  memset(P, 0, sizeof(double) * (size_t)(T * T));
  memset(dP, 0, sizeof(double) * (size_t)(T * T));
  memset(dS, 0, sizeof(double) * (size_t)(T * T));
  for (long i = 0; i < T; ++i) {
    softmax_row(i, D, s, q, k, p);
    for (long j = 0; j <= i; ++j) {
      double dp = 0.0;
      for (long d = 0; d < D; ++d) dp += dout[i * D + d] * v[j * D + d];
      P[i * T + j] = p[j];
      dP[i * T + j] = dp;
      dS[i * T + j] = p[j] * (dp - delta[i]);
    }
  }
  free(o);
  free(p);
  return ORACLE_OK;
}

/* ==== attention dropout ===================================================
 *
 * nanoGPT passes dropout_p = its dropout rate to the fused attention call in
 * training (page "nanoGPT: a real GPT in two 300-line files", section 2 "How
 * the code works"): every attention weight P_ij is zeroed with probability
 * p and the survivors are scaled by 1/(1-p), after the softmax and before
 * the product with V.
 *
 * With a keep mask M (M_ij in {0, 1}) and z = 1/(1-p):
 *   Pd_ij  = z M_ij P_ij,            O_i = sum_j Pd_ij V_j
 *   LSE_i  as without dropout (the softmax is unchanged)
 * Backward, the chain rule through the same three steps:
 *   dPd_ij = sum_d dO_id V_jd,       dV_j = sum_i Pd_ij dO_i
 *   dP_ij  = z M_ij dPd_ij
 *   dS_ij  = P_ij (dP_ij - sum_k P_ik dP_ik)   (softmax Jacobian)
 *   dQ_i   = s sum_j dS_ij K_j,      dK_j = s sum_i dS_ij Q_i
 *
 * The mask. The pages fix no generator; the one used here is
 * Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11, section 4), a keyed bijection on 128-bit counters.
 * For head bh (= b*H + h), query i, key j, with a 64-bit seed and a 32-bit
 * offset (a caller-chosen stream number):
 *   key     = (seed mod 2^32, seed div 2^32)
 *   counter = (j div 8, i, bh, offset)
 *   u_ij    = 16-bit field (j mod 2) of output word (j mod 8) div 2
 *   thr     = round(p * 65536),  M_ij = [u_ij >= thr]
 * so a dropped weight has probability thr/65536 (p rounded to a multiple of
 * 2^-16), and z = 65536 / (65536 - thr) keeps E[z M] = 1 exactly.
 */

/* Philox4x32 with 10 rounds. One round: two 32x32 -> 64-bit products of
 * counter words 0 and 2 with the round multipliers; the new words are
 * (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0)). Between
 * rounds the key words are bumped by the Weyl constants (the golden ratio
 * and sqrt(3) - 1 in 32-bit fixed point). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * x0;
    const uint64_t p1 = (uint64_t)M1 * x2;
    const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
    const uint32_t y1 = (uint32_t)p1;
    const uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
    const uint32_t y3 = (uint32_t)p0;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
    k0 += W0;
    k1 += W1;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* thr = round(p * 65536) for 0 <= p < 1, or -1 when p is outside [0, 1) or
 * rounds to 65536 (everything dropped). */
long oracle_dropout_threshold(double p) {
  if (!(p >= 0.0 && p < 1.0)) return -1;
  const double t = floor(p * 65536.0 + 0.5);
  return t >= 65536.0 ? -1 : (long)t;
}

/* Keep mask [n, T, T] (uint8, 1 = kept; zero above the diagonal) of the heads
 * listed in bh[0..n-1] (flat b*H + h indices). */
int oracle_dropout_keep(long n, const long* bh, long T, double p, uint64_t seed,
                        uint32_t offset, uint8_t* keep) {
  const long thr = oracle_dropout_threshold(p);
  if (n < 0 || T < 0 || thr < 0 || (n > 0 && (!bh || !keep))) return ORACLE_EINVAL;
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (long h = 0; h < n; ++h) {
    uint8_t* mh = keep + h * T * T;
    memset(mh, 0, (size_t)(T * T));
    for (long i = 0; i < T; ++i)
      for (long j = 0; j <= i; ++j) {
        const uint32_t ctr[4] = {(uint32_t)(j / 8), (uint32_t)i, (uint32_t)bh[h], offset};
        uint32_t out[4];
        oracle_philox4x32_10(ctr, key, out);
        const uint32_t word = out[(j % 8) / 2];
        const uint32_t u = (word >> (16 * (j % 2))) & 0xFFFFu;
        mh[i * T + j] = u >= (uint32_t)thr ? 1 : 0;
      }
  }
  return ORACLE_OK;
}

/* One head, forward with dropout. p is T doubles of scratch. */
static void head_forward_dropout(long T, long D, const double* q, const double* k,
                                 const double* v, const uint8_t* M, double z, double* o,
                                 double* lse, double* p) {
  const double s = 1.0 / sqrt((double)D);
  for (long i = 0; i < T; ++i) {
    const double li = softmax_row(i, D, s, q, k, p);
    if (lse) lse[i] = li;
    double* oi = o + i * D;
    for (long d = 0; d < D; ++d) oi[d] = 0.0;
    for (long j = 0; j <= i; ++j) {
      const double pd = M[i * T + j] ? z * p[j] : 0.0;
      const double* vj = v + j * D;
      for (long d = 0; d < D; ++d) oi[d] += pd * vj[d];
    }
  }
}

/* One head, backward with dropout. p and dp are T doubles of scratch. */
static void head_backward_dropout(long T, long D, const double* q, const double* k,
                                  const double* v, const double* dout, const uint8_t* M,
                                  double z, double* dq, double* dk, double* dv, double* p,
                                  double* dp) {
  const double s = 1.0 / sqrt((double)D);
  memset(dq, 0, sizeof(double) * T * D);
  memset(dk, 0, sizeof(double) * T * D);
  memset(dv, 0, sizeof(double) * T * D);
  for (long i = 0; i < T; ++i) {
    softmax_row(i, D, s, q, k, p);
    const double* qi = q + i * D;
    const double* doi = dout + i * D;
    double* dqi = dq + i * D;
    double rowdot = 0.0; /* sum_k P_ik dP_ik */
    for (long j = 0; j <= i; ++j) {
      const double* vj = v + j * D;
      double dpd = 0.0;
      for (long d = 0; d < D; ++d) dpd += doi[d] * vj[d];
      dp[j] = M[i * T + j] ? z * dpd : 0.0;
      rowdot += p[j] * dp[j];
      const double pd = M[i * T + j] ? z * p[j] : 0.0;
      double* dvj = dv + j * D;
      for (long d = 0; d < D; ++d) dvj[d] += pd * doi[d];
    }
    for (long j = 0; j <= i; ++j) {
      const double ds = p[j] * (dp[j] - rowdot);
      const double* kj = k + j * D;
      double* dkj = dk + j * D;
      for (long d = 0; d < D; ++d) {
        dqi[d] += s * ds * kj[d];
        dkj[d] += s * ds * qi[d];
      }
    }
  }
}

typedef struct {
  int backward;
  long heads, T, D;
  const double *q, *k, *v, *dout;
  const uint8_t* keep;
  double z;
  double *o, *lse, *dq, *dk, *dv;
  int tid, nthreads, status;
} djob_t;

static void* run_djob(void* arg) {
  djob_t* jb = (djob_t*)arg;
  const long T = jb->T, D = jb->D, E = T * D;
  double* p = (double*)malloc(sizeof(double) * (size_t)T);
  double* dp = (double*)malloc(sizeof(double) * (size_t)T);
  if (!p || !dp) {
    jb->status = ORACLE_ENOMEM;
  } else {
    for (long h = jb->tid; h < jb->heads; h += jb->nthreads) {
      const uint8_t* M = jb->keep + h * T * T;
      if (jb->backward)
        head_backward_dropout(T, D, jb->q + h * E, jb->k + h * E, jb->v + h * E,
                              jb->dout + h * E, M, jb->z, jb->dq + h * E, jb->dk + h * E,
                              jb->dv + h * E, p, dp);
      else
        head_forward_dropout(T, D, jb->q + h * E, jb->k + h * E, jb->v + h * E, M, jb->z,
                             jb->o + h * E, jb->lse ? jb->lse + h * T : NULL, p);
    }
    jb->status = ORACLE_OK;
  }
  free(p);
  free(dp);
  return NULL;
}

static int run_djobs(djob_t proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 1024) nthreads = 1024;
  if ((long)nthreads > proto.heads) nthreads = (int)(proto.heads > 0 ? proto.heads : 1);
  djob_t* jobs = (djob_t*)calloc((size_t)nthreads, sizeof(djob_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return ORACLE_ENOMEM;
  }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].tid = t;
    jobs[t].nthreads = nthreads;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, run_djob, &jobs[t]) != 0) break;
    started = t;
  }
  run_djob(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; ++t) run_djob(&jobs[t]);
  int status = ORACLE_OK;
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != ORACLE_OK) status = jobs[t].status;
  free(jobs);
  free(th);
  return status;
}

/* Forward with dropout: keep [heads, T, T] (uint8) and z = 1/(1-p). */
int oracle_attn_fwd_dropout(long heads, long T, long D, const double* q, const double* k,
                            const double* v, const uint8_t* keep, double z, double* o,
                            double* lse, int nthreads) {
  if (heads < 0 || T < 0 || D < 1 || !q || !k || !v || !keep || !o) return ORACLE_EINVAL;
  if (heads == 0 || T == 0) return ORACLE_OK;
  djob_t jb;
  memset(&jb, 0, sizeof jb);
  jb.heads = heads;
  jb.T = T;
  jb.D = D;
  jb.q = q;
  jb.k = k;
  jb.v = v;
  jb.keep = keep;
  jb.z = z;
  jb.o = o;
  jb.lse = lse;
  return run_djobs(jb, nthreads);
}

/* Backward with dropout: gradients of sum(dout * O) for the forward above. */
int oracle_attn_bwd_dropout(long heads, long T, long D, const double* q, const double* k,
                            const double* v, const double* dout, const uint8_t* keep,
                            double z, double* dq, double* dk, double* dv, int nthreads) {
  if (heads < 0 || T < 0 || D < 1 || !q || !k || !v || !dout || !keep || !dq || !dk || !dv)
    return ORACLE_EINVAL;
  if (heads == 0 || T == 0) return ORACLE_OK;
  djob_t jb;
  memset(&jb, 0, sizeof jb);
  jb.backward = 1;
  jb.heads = heads;
  jb.T = T;
  jb.D = D;
  jb.q = q;
  jb.k = k;
  jb.v = v;
  jb.dout = dout;
  jb.keep = keep;
  jb.z = z;
  jb.dq = dq;
  jb.dk = dk;
  jb.dv = dv;
  return run_djobs(jb, nthreads);
}

/* ==== one query against a key/value cache ================================
 *
 * Sampling (generate() on the same page, section 2) feeds the sequence back
 * one position at a time; the newest position's query attends to every key
 * up to and including its own. With a cache of n keys and values that is the
 * last row of the causal forward at T = n:
 *   S_j = s q.K_j (j < n),  O = sum_j softmax(S)_j V_j,  LSE = ln sum_j e^S_j
 * heads are independent; each head h has its own length n_h (0 <= n_h <= L,
 * cache rows beyond n_h are ignored). n_h = 0 gives O = 0 and LSE = -inf.
 * q is [heads, D], the caches [heads, L, D], o [heads, D], lse [heads].
 */
int oracle_attn_decode(long heads, long L, long D, const double* q, const double* k,
                       const double* v, const long* lengths, double* o, double* lse) {
  if (heads < 0 || L < 0 || D < 1 || (heads > 0 && (!q || !k || !v || !lengths || !o || !lse)))
    return ORACLE_EINVAL;
  const double s = 1.0 / sqrt((double)D);
  double* p = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  if (!p) return ORACLE_ENOMEM;
  for (long h = 0; h < heads; ++h) {
    const long n = lengths[h];
    if (n < 0 || n > L) {
      free(p);
      return ORACLE_EINVAL;
    }
    const double* qh = q + h * D;
    const double* kh = k + h * L * D;
    const double* vh = v + h * L * D;
    double* oh = o + h * D;
    for (long d = 0; d < D; ++d) oh[d] = 0.0;
    if (n == 0) {
      lse[h] = -INFINITY;
      continue;
    }
    double m = -INFINITY;
    for (long j = 0; j < n; ++j) {
      double dot = 0.0;
      for (long d = 0; d < D; ++d) dot += qh[d] * kh[j * D + d];
      p[j] = s * dot;
      if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (long j = 0; j < n; ++j) {
      p[j] = exp(p[j] - m);
      l += p[j];
    }
    for (long j = 0; j < n; ++j)
      for (long d = 0; d < D; ++d) oh[d] += (p[j] / l) * vh[j * D + d];
    lse[h] = m + log(l);
  }
  free(p);
  return ORACLE_OK;
}

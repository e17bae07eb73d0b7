/*
 * gdn2_oracle.c -- fp64 CPU oracle for the Gated DeltaNet-2 forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library.
 *
 * It is the plain definition, one token at a time, in double precision.
 * For every sequence n and value head h (query/key head g = h / (H_v / H_qk)):
 *
 *   S <- S0[n, h]  (or zeros)
 *   for t = 0 .. T-1:
 *     1. decay:  S[i][j] *= a[t][i]
 *        (channel-wise decay on the key axis, applied to the previous state
 *         before anything else: Gated DeltaNet-2 post on tilnote.io, section
 *         on the GDN-2 design; the delta-rule tutorial on ai-systems-
 *         engineering.com announces the keep-how-much step ahead of the
 *         correction in its closing section)
 *     2. k-read: r[j] = sum_i S[i][j] * k[t][i]
 *        (read the current state with the key before changing it: tutorial,
 *         "record the difference" section, r^T = k^T S, and the key-versus-
 *         query table)
 *     3. erase:  S[i][j] -= b[t][i] * k[t][i] * r[j]
 *        (remove the key-side component, gated channel-wise by b on the key
 *         axis: tilnote GDN-2 design section; news.hamidun.com architecture
 *         section)
 *     4. write:  S[i][j] += k[t][i] * w[t][j] * v[t][j]
 *        (add the value-side component, gated channel-wise by w on the value
 *         axis: same two passages)
 *     5. read:   o[t][j] = sum_i S[i][j] * q[t][i]
 *        (the query reads the updated state, so the output covers the current
 *         token: tutorial, "write with KV, read with Q" section and its
 *         figure 1)
 *   S_T[n, h] <- S
 *
 * State orientation: rows are key channels and columns are value channels,
 * so a read is x^T S and a write adds an outer product k y^T (tutorial,
 * "record the difference" section). No score normalisation and no query
 * scale are applied (tutorial, key-versus-query section).
 *
 * Steps 3 and 4 are the plainest reading of the prose description of the
 * decoupled gates; the pages give no formula for them. With b = w = beta
 * (uniform) and a = 1 they reduce to the delta rule S + beta k (v - S^T k)^T
 * of the tutorial's beta section.
 *
 * Layouts (row-major, contiguous), all double:
 *   q, k : [B, T, H_qk, d_k]     v, w : [B, T, H_v, d_v]
 *   a, b : [B, T, H_v, d_k]      S0, S_T : [B, H_v, d_k, d_v]   o : [B, T, H_v, d_v]
 * S0 may be NULL (zero state); S_T may be NULL (not written) and may alias S0.
 *
 * Build: gcc -O2 -fPIC -shared (no fast-math), pthreads across (n, h) pairs.
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

typedef struct {
  int B, T, Hqk, Hv, dk, dv;
  const double *q, *k, *v, *a, *b, *w, *S0;
  double *o, *ST;
  int next_unit;        /* next (n, h) pair to process */
  pthread_mutex_t lock;
  int fail;
} job_t;

static void run_unit(const job_t *J, int unit, double *S, double *r) {
  const int n = unit / J->Hv, h = unit % J->Hv;
  const int G = J->Hv / J->Hqk, g = h / G;
  const int dk = J->dk, dv = J->dv;
  const size_t qk_tok = (size_t)J->Hqk * dk;   /* stride of one token in q, k */
  const size_t ab_tok = (size_t)J->Hv * dk;    /* ... in a, b */
  const size_t vw_tok = (size_t)J->Hv * dv;    /* ... in v, w, o */
  const size_t s_off = ((size_t)n * J->Hv + h) * (size_t)dk * dv;

  if (J->S0)
    memcpy(S, J->S0 + s_off, sizeof(double) * (size_t)dk * dv);
  else
    memset(S, 0, sizeof(double) * (size_t)dk * dv);

  for (int t = 0; t < J->T; ++t) {
    const size_t tok = (size_t)n * J->T + t;
    const double *qt = J->q + tok * qk_tok + (size_t)g * dk;
    const double *kt = J->k + tok * qk_tok + (size_t)g * dk;
    const double *at = J->a + tok * ab_tok + (size_t)h * dk;
    const double *bt = J->b + tok * ab_tok + (size_t)h * dk;
    const double *vt = J->v + tok * vw_tok + (size_t)h * dv;
    const double *wt = J->w + tok * vw_tok + (size_t)h * dv;
    double *ot = J->o ? J->o + tok * vw_tok + (size_t)h * dv : NULL;

    /* 1. decay the key-axis rows */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= at[i];
    /* 2. read the decayed state with the key */
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) r[j] += S[(size_t)i * dv + j] * kt[i];
    /* 3. erase the key-side component, gated by b on the key axis
     * 4. write the value-side component, gated by w on the value axis */
    for (int i = 0; i < dk; ++i) {
      const double e = bt[i] * kt[i];
      for (int j = 0; j < dv; ++j) {
        S[(size_t)i * dv + j] -= e * r[j];
        S[(size_t)i * dv + j] += kt[i] * (wt[j] * vt[j]);
      }
    }
    /* 5. the query reads the updated state */
    if (ot) {
      for (int j = 0; j < dv; ++j) ot[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];
    }
  }
  if (J->ST) memcpy(J->ST + s_off, S, sizeof(double) * (size_t)dk * dv);
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  double *S = (double *)malloc(sizeof(double) * (size_t)J->dk * J->dv);
  double *r = (double *)malloc(sizeof(double) * (size_t)J->dv);
  if (!S || !r) {
    pthread_mutex_lock(&J->lock);
    J->fail = 1;
    pthread_mutex_unlock(&J->lock);
    free(S);
    free(r);
    return NULL;
  }
  const int units = J->B * J->Hv;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const int u = J->next_unit++;
    pthread_mutex_unlock(&J->lock);
    if (u >= units) break;
    run_unit(J, u, S, r);
  }
  free(S);
  free(r);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure.
 * If elapsed_s is non-NULL it receives the wall time of the recurrence alone. */
int gdn2_oracle_forward(int B, int T, int Hqk, int Hv, int dk, int dv,
                        const double *q, const double *k, const double *v,
                        const double *a, const double *b, const double *w,
                        const double *S0, double *o, double *ST,
                        int nthreads, double *elapsed_s) {
  if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return -1;
  if (Hv % Hqk != 0) return -1;
  if (T > 0 && (!q || !k || !v || !a || !b || !w)) return -1;
  job_t J;
  J.B = B; J.T = T; J.Hqk = Hqk; J.Hv = Hv; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.a = a; J.b = b; J.w = w; J.S0 = S0;
  J.o = o; J.ST = ST;
  J.next_unit = 0;
  J.fail = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > B * Hv) nthreads = B * Hv > 0 ? B * Hv : 1;

  struct timespec t0, t1;
  clock_gettime(CLOCK_MONOTONIC, &t0);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  if (th) {
    for (int i = 0; i < nthreads; ++i) {
      if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
      ++started;
    }
  }
  if (started == 0) worker(&J); /* run inline */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  clock_gettime(CLOCK_MONOTONIC, &t1);
  free(th);
  pthread_mutex_destroy(&J.lock);
  if (elapsed_s)
    *elapsed_s = (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
  return J.fail ? -2 : 0;
}

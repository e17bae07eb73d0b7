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

/*
 * Backward pass (gradients of the same recurrence), fp64.
 *
 * The pages define no backward pass; training the layer (the GDN-2 post on
 * tilnote.io reports a 1.3B-parameter model trained on 100B tokens) needs
 * the derivative of the forward map above. This is reverse-mode
 * differentiation of steps 1-5, one token at a time from the last token to
 * the first, with every state S_t kept from a forward run (no recomputation
 * tricks). Given upstream gradients dO = dL/do and dS_T = dL/dS_T (NULL:
 * zero), with L the running adjoint dL/dS of the state after token t:
 *
 *   5. read:   dq_t[i] = sum_j S_t[i][j] dO_t[j];   L[i][j] += q_t[i] dO_t[j]
 *   4./3. with e = b_t*k_t, u = w_t*v_t and r the k-read of step 2:
 *              du[j] = sum_i L[i][j] k_t[i]  -> dv_t[j] = du[j] w_t[j], dw_t[j] = du[j] v_t[j]
 *              de[i] = -sum_j L[i][j] r[j]   -> db_t[i] = de[i] k_t[i],  dk_t[i] += de[i] b_t[i]
 *              dk_t[i] += sum_j L[i][j] u[j]
 *              dr[j] = -sum_i L[i][j] e[i]
 *   2. k-read (r = Sd^T k, Sd the decayed state):
 *              dk_t[i] += sum_j Sd[i][j] dr[j];  L[i][j] += k_t[i] dr[j]   (L is now dL/dSd)
 *   1. decay (Sd = diag(a_t) S_{t-1}):
 *              da_t[i] = sum_j L[i][j] S_{t-1}[i][j];  L[i][j] *= a_t[i]
 *
 * and finally dS0 = L. dq and dk are returned per value head
 * ([B, T, H_v, d_k]); the QK-head gradient is their sum over the value heads
 * that share the QK head (done by the caller).
 */
typedef struct {
  int B, T, Hqk, Hv, dk, dv;
  const double *q, *k, *v, *a, *b, *w, *S0, *dO, *dST;
  double *dq, *dk_, *dv_, *da, *db, *dw, *dS0;
  int next_unit;
  pthread_mutex_t lock;
  int fail;
} bjob_t;

static void run_unit_bwd(const bjob_t *J, int unit, double *hist, double *rs, double *L, double *du,
                         double *dr) {
  const int n = unit / J->Hv, h = unit % J->Hv;
  const int grp = J->Hv / J->Hqk, g = h / grp;
  const int dk = J->dk, dv = J->dv, T = J->T;
  const size_t qk_tok = (size_t)J->Hqk * dk, ab_tok = (size_t)J->Hv * dk, vw_tok = (size_t)J->Hv * dv;
  const size_t ssz = (size_t)dk * dv;
  const size_t s_off = ((size_t)n * J->Hv + h) * ssz;

  /* forward: hist[t + 1] = S after token t, hist[0] = S0; rs[t] = k-read */
  if (J->S0)
    memcpy(hist, J->S0 + s_off, sizeof(double) * ssz);
  else
    memset(hist, 0, sizeof(double) * ssz);
  for (int t = 0; t < T; ++t) {
    const size_t tok = (size_t)n * T + t;
    const double *kt = J->k + tok * qk_tok + (size_t)g * dk;
    const double *at = J->a + tok * ab_tok + (size_t)h * dk;
    const double *bt = J->b + tok * ab_tok + (size_t)h * dk;
    const double *vt = J->v + tok * vw_tok + (size_t)h * dv;
    const double *wt = J->w + tok * vw_tok + (size_t)h * dv;
    const double *Sp = hist + (size_t)t * ssz;
    double *Sn = hist + (size_t)(t + 1) * ssz;
    double *rt = rs + (size_t)t * dv;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] = Sp[(size_t)i * dv + j] * at[i];
    for (int j = 0; j < dv; ++j) rt[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) rt[j] += Sn[(size_t)i * dv + j] * kt[i];
    for (int i = 0; i < dk; ++i) {
      const double eb = bt[i] * kt[i];
      for (int j = 0; j < dv; ++j) {
        Sn[(size_t)i * dv + j] -= eb * rt[j];
        Sn[(size_t)i * dv + j] += (wt[j] * vt[j]) * kt[i];
      }
    }
  }

  /* backward */
  if (J->dST)
    memcpy(L, J->dST + s_off, sizeof(double) * ssz);
  else
    memset(L, 0, sizeof(double) * ssz);
  for (int t = T - 1; t >= 0; --t) {
    const size_t tok = (size_t)n * T + t;
    const double *qt = J->q + tok * qk_tok + (size_t)g * dk;
    const double *kt = J->k + tok * qk_tok + (size_t)g * dk;
    const double *at = J->a + tok * ab_tok + (size_t)h * dk;
    const double *bt = J->b + tok * ab_tok + (size_t)h * dk;
    const double *vt = J->v + tok * vw_tok + (size_t)h * dv;
    const double *wt = J->w + tok * vw_tok + (size_t)h * dv;
    const double *dOt = J->dO + tok * vw_tok + (size_t)h * dv;
    const double *St = hist + (size_t)(t + 1) * ssz;
    const double *Sp = hist + (size_t)t * ssz;
    const double *r = rs + (size_t)t * dv;
    double *dqt = J->dq + tok * ab_tok + (size_t)h * dk;
    double *dkt = J->dk_ + tok * ab_tok + (size_t)h * dk;
    double *dat = J->da + tok * ab_tok + (size_t)h * dk;
    double *dbt = J->db + tok * ab_tok + (size_t)h * dk;
    double *dvt = J->dv_ + tok * vw_tok + (size_t)h * dv;
    double *dwt = J->dw + tok * vw_tok + (size_t)h * dv;

    /* 5. the query read o_t = S_t^T q_t */
    for (int i = 0; i < dk; ++i) {
      double s = 0.0;
      for (int j = 0; j < dv; ++j) s += St[(size_t)i * dv + j] * dOt[j];
      dqt[i] = s;
    }
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += qt[i] * dOt[j];
    /* 4. write k u^T and 3. erase e r^T */
    for (int j = 0; j < dv; ++j) {
      du[j] = 0.0;
      dr[j] = 0.0;
    }
    for (int i = 0; i < dk; ++i) {
      const double eb = bt[i] * kt[i];
      for (int j = 0; j < dv; ++j) {
        du[j] += L[(size_t)i * dv + j] * kt[i];
        dr[j] -= L[(size_t)i * dv + j] * eb;
      }
    }
    for (int j = 0; j < dv; ++j) {
      dvt[j] = du[j] * wt[j];
      dwt[j] = du[j] * vt[j];
    }
    for (int i = 0; i < dk; ++i) {
      double de = 0.0, kw = 0.0;
      for (int j = 0; j < dv; ++j) {
        de -= L[(size_t)i * dv + j] * r[j];
        kw += L[(size_t)i * dv + j] * (wt[j] * vt[j]);
      }
      dbt[i] = de * kt[i];
      dkt[i] = kw + de * bt[i];
    }
    /* 2. the k-read r = Sd^T k, Sd = diag(a_t) S_{t-1} */
    for (int i = 0; i < dk; ++i) {
      double s = 0.0;
      for (int j = 0; j < dv; ++j) s += at[i] * Sp[(size_t)i * dv + j] * dr[j];
      dkt[i] += s;
      for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] += kt[i] * dr[j];
    }
    /* 1. the decay */
    for (int i = 0; i < dk; ++i) {
      double s = 0.0;
      for (int j = 0; j < dv; ++j) s += L[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
      dat[i] = s;
      for (int j = 0; j < dv; ++j) L[(size_t)i * dv + j] *= at[i];
    }
  }
  if (J->dS0) memcpy(J->dS0 + s_off, L, sizeof(double) * ssz);
}

static void *worker_bwd(void *arg) {
  bjob_t *J = (bjob_t *)arg;
  const size_t ssz = (size_t)J->dk * J->dv;
  double *hist = (double *)malloc(sizeof(double) * ssz * ((size_t)J->T + 1));
  double *rs = (double *)malloc(sizeof(double) * (size_t)J->dv * ((size_t)J->T + 1));
  double *L = (double *)malloc(sizeof(double) * ssz);
  double *du = (double *)malloc(sizeof(double) * (size_t)J->dv);
  double *dr = (double *)malloc(sizeof(double) * (size_t)J->dv);
  if (!hist || !rs || !L || !du || !dr) {
    pthread_mutex_lock(&J->lock);
    J->fail = 1;
    pthread_mutex_unlock(&J->lock);
  } else {
    const int units = J->B * J->Hv;
    for (;;) {
      pthread_mutex_lock(&J->lock);
      const int u = J->next_unit++;
      pthread_mutex_unlock(&J->lock);
      if (u >= units) break;
      run_unit_bwd(J, u, hist, rs, L, du, dr);
    }
  }
  free(hist);
  free(rs);
  free(L);
  free(du);
  free(dr);
  return NULL;
}

/* Gradients of the forward map. Layouts as the forward, plus dO like o and
 * dS_T like S_T (NULL: zero). Outputs: dq, dk per value head [B, T, H_v, d_k];
 * dv, dw [B, T, H_v, d_v]; da, db [B, T, H_v, d_k]; dS0 [B, H_v, d_k, d_v]
 * (NULL: not written). Each worker thread holds T + 1 states of one head.
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int gdn2_oracle_backward(int B, int T, int Hqk, int Hv, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *a, const double *b, const double *w,
                         const double *S0, const double *dO, const double *dST,
                         double *dq, double *dk_out, double *dv_out, double *da, double *db,
                         double *dw, double *dS0, int nthreads) {
  if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return -1;
  if (Hv % Hqk != 0) return -1;
  if (T > 0 && (!q || !k || !v || !a || !b || !w || !dO || !dq || !dk_out || !dv_out || !da || !db || !dw))
    return -1;
  bjob_t J;
  J.B = B; J.T = T; J.Hqk = Hqk; J.Hv = Hv; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.a = a; J.b = b; J.w = w; J.S0 = S0; J.dO = dO; J.dST = dST;
  J.dq = dq; J.dk_ = dk_out; J.dv_ = dv_out; J.da = da; J.db = db; J.dw = dw; J.dS0 = dS0;
  J.next_unit = 0;
  J.fail = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > B * Hv) nthreads = B * Hv > 0 ? B * Hv : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  if (th) {
    for (int i = 0; i < nthreads; ++i) {
      if (pthread_create(&th[i], NULL, worker_bwd, &J) != 0) break;
      ++started;
    }
  }
  if (started == 0) worker_bwd(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return J.fail ? -2 : 0;
}

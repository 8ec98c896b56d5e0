/*
 * Gated DeltaNet oracle: plain fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it. It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (all in double precision, token by token, no chunking):
 *
 *   Gated delta rule, per head (page "NLP——技术报告解读-Qwen3.8-Flash-Next",
 *   section "Gated DeltaNet 核心机制", the update-rule display):
 *     decayed state      St  = alpha_t * S_{t-1}
 *     prediction error   e_t = v_t - St^T k_t
 *     write              S_t = St + beta_t * k_t e_t^T
 *     read               y_t = S_t^T q_t
 *   The same page gives the equivalent closed form
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *   implemented separately (form = GDN_ORACLE_FORM_CLOSED) so the two can
 *   be checked against each other.
 *
 *   Front end (same page, section "GDN 参数化细节", first display; the paper's
 *   Fig. 2 caption on the pwwt.cn page calls the convolution short and
 *   causal): q = L2Norm(SiLU(ShortConv(x_q))), k likewise, v = SiLU(ShortConv(x_v)).
 *
 *   Output gate (same section, third display; zero-centred RMSNorm from the
 *   pwwt.cn page, section 2.1.1): o = sigmoid(z) * RMSNorm(y) with gain 1 + w.
 *
 *   Backward (gradients of the recurrence above; the pages report backward
 *   kernels but print no formula, so this is reverse-mode differentiation of
 *   the erase-write form written out by hand, token by token, from the last
 *   token to the first). With S~ = alpha S_{t-1}, e = v - S~^T k:
 *     dq_t = S_t dy_t,              dS += q dy^T,
 *     dbeta = k^T dS e,             de = beta dS^T k,
 *     dk = beta dS e - S~ de,       dv = de,
 *     dS~ = dS - k de^T,            dlog_alpha = alpha <S_{t-1}, dS~>,
 *     dS <- alpha dS~  (the gradient of S_{t-1}); dS0 is dS after token 1.
 *
 *   Gates from raw pre-activations (same section, second display):
 *   beta_t = sigmoid(b_t), alpha_t = exp[-exp(A) softplus(a_t + b_alpha)],
 *   i.e. log alpha_t = -exp(A) * softplus(a_t + b_alpha), per head.
 *
 * Layouts (row-major, token-major):
 *   q, k        [sum_T, H, dk]
 *   v, y, z, o  [sum_T, H, dv]
 *   log_alpha, beta [sum_T, H]
 *   S0, S_T, S  [N, H, dk, dv]
 *   cu_seqlens  int32[N+1] (NULL: N sequences of T tokens each)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GDN_ORACLE_FORM_ERASE_WRITE 0
#define GDN_ORACLE_FORM_CLOSED 1

static int64_t seq_start(const int32_t *cu, int n, int T) {
  return cu ? (int64_t)cu[n] : (int64_t)n * T;
}
static int64_t seq_len(const int32_t *cu, int n, int T) {
  return cu ? (int64_t)(cu[n + 1] - cu[n]) : (int64_t)T;
}

/* One (sequence, head, column block) of the recurrence. S points to a
 * dk x dv row-major state; only columns [c0, c1) are touched, which is
 * legitimate because every column of S evolves on its own: the update of
 * column j reads only column j, k_t, v_t[j] and the gates. */
static void run_unit(const double *q, const double *k, const double *v,
                     const double *log_alpha, const double *beta, double *S,
                     double *y, int64_t t0, int64_t len, int h, int H, int dk,
                     int dv, int c0, int c1, int form) {
  double *u = (double *)malloc(sizeof(double) * (size_t)dv);
  for (int64_t t = t0; t < t0 + len; ++t) {
    const double *qt = q + (t * H + h) * dk;
    const double *kt = k + (t * H + h) * dk;
    const double *vt = v + (t * H + h) * dv;
    const double a = exp(log_alpha[t * H + h]);
    const double b = beta[t * H + h];
    if (form == GDN_ORACLE_FORM_ERASE_WRITE) {
      /* decay first */
      for (int i = 0; i < dk; ++i)
        for (int j = c0; j < c1; ++j) S[i * dv + j] *= a;
      /* e = v - S~^T k */
      for (int j = c0; j < c1; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kt[i];
        u[j] = vt[j] - acc;
      }
      /* S = S~ + beta k e^T */
      for (int i = 0; i < dk; ++i)
        for (int j = c0; j < c1; ++j) S[i * dv + j] += b * kt[i] * u[j];
    } else {
      /* u = k^T S_{t-1} (row vector over columns) */
      for (int j = c0; j < c1; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += kt[i] * S[i * dv + j];
        u[j] = acc;
      }
      /* S = a (S - b k u) + b k v^T */
      for (int i = 0; i < dk; ++i)
        for (int j = c0; j < c1; ++j)
          S[i * dv + j] =
              a * (S[i * dv + j] - b * kt[i] * u[j]) + b * kt[i] * vt[j];
    }
    /* y = S_t^T q */
    double *yt = y ? y + (t * H + h) * dv : NULL;
    if (yt) {
      for (int j = c0; j < c1; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];
        yt[j] = acc;
      }
    }
  }
  free(u);
}

/* Full-sequence recurrence. y may be NULL (state only). S_T must be given.
 * col_blocks >= 1 splits the dv columns into that many independent pieces
 * for parallelism; the result does not depend on it. Returns 0 on success. */
int oracle_gdn_fwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta,
                   const double *S0, double *y, double *S_T,
                   const int32_t *cu_seqlens, int N, int T, int H, int dk,
                   int dv, int form, int nthreads, int col_blocks) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S_T) return -1;
  if (col_blocks < 1) col_blocks = 1;
  if (col_blocks > dv) col_blocks = dv;
  const size_t state = (size_t)dk * dv;
  for (int64_t u = 0; u < (int64_t)N * H; ++u) {
    if (S0)
      memcpy(S_T + u * state, S0 + u * state, sizeof(double) * state);
    else
      memset(S_T + u * state, 0, sizeof(double) * state);
  }
  const int64_t units = (int64_t)N * H * col_blocks;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t w = 0; w < units; ++w) {
    const int cb = (int)(w % col_blocks);
    const int64_t nh = w / col_blocks;
    const int h = (int)(nh % H);
    const int n = (int)(nh / H);
    const int c0 = (int)((int64_t)dv * cb / col_blocks);
    const int c1 = (int)((int64_t)dv * (cb + 1) / col_blocks);
    run_unit(q, k, v, log_alpha, beta, S_T + nh * state, y,
             seq_start(cu_seqlens, n, T), seq_len(cu_seqlens, n, T), h, H, dk,
             dv, c0, c1, form);
  }
  return 0;
}

/* Single-token decode: one step of the recurrence applied in place to S
 * [N, H, dk, dv]; q, k [N, H, dk], v and y [N, H, dv], gates [N, H]. */
int oracle_decode_step(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *beta, double *S,
                       double *y, int N, int H, int dk, int dv, int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S) return -1;
  const size_t state = (size_t)dk * dv;
  const int64_t units = (int64_t)N * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
  for (int64_t nh = 0; nh < units; ++nh) {
    const int h = (int)(nh % H);
    const int n = (int)(nh / H);
    run_unit(q, k, v, log_alpha, beta, S + nh * state, y, (int64_t)n, 1, h, H,
             dk, dv, 0, dv, GDN_ORACLE_FORM_ERASE_WRITE);
  }
  return 0;
}

/* Front end for one projected stream x [sum_T, H, d]:
 *   u_t[c] = sum_{j=0..K-1} w[c][j] * x_{t-(K-1)+j}[c]   (causal, no bias,
 *            history before the sequence start is zero)
 *   a_t    = SiLU(u_t) = u_t / (1 + exp(-u_t))
 *   out_t  = a_t * (sum_c a_t[c]^2 + eps)^(-1/2) over the head's d channels
 *            when l2 != 0, else a_t.
 * Channel c = h * d + i; w is [H * d][K]. */
int oracle_frontend(const double *x, const double *w, double *out,
                    const int32_t *cu_seqlens, int N, int T, int H, int d,
                    int K, int l2, double eps, int nthreads) {
  if (N < 0 || H <= 0 || d <= 0 || K <= 0) return -1;
  const int64_t units = (int64_t)N * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t nh = 0; nh < units; ++nh) {
    const int h = (int)(nh % H);
    const int n = (int)(nh / H);
    const int64_t t0 = seq_start(cu_seqlens, n, T);
    const int64_t len = seq_len(cu_seqlens, n, T);
    double *a = (double *)malloc(sizeof(double) * (size_t)d);
    for (int64_t t = 0; t < len; ++t) {
      for (int i = 0; i < d; ++i) {
        const int64_t c = (int64_t)h * d + i;
        double acc = 0.0;
        for (int j = 0; j < K; ++j) {
          const int64_t src = t - (K - 1) + j;
          if (src < 0) continue; /* zero history at the sequence start */
          acc += w[c * K + j] * x[((t0 + src) * H + h) * d + i];
        }
        a[i] = acc / (1.0 + exp(-acc));
      }
      double scale = 1.0;
      if (l2) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += a[i] * a[i];
        scale = 1.0 / sqrt(ss + eps);
      }
      for (int i = 0; i < d; ++i)
        out[((t0 + t) * H + h) * d + i] = a[i] * scale;
    }
    free(a);
  }
  return 0;
}

/* Output gate per (token, head) row of d values:
 *   o = sigmoid(z) * y * (mean(y^2) + eps)^(-1/2) * (1 + w)
 * w [d] is the zero-centred RMSNorm weight shared by all heads (may be
 * NULL: w = 0). */
int oracle_output_gate(const double *y, const double *z, const double *w,
                       double eps, double *o, int64_t rows, int d,
                       int nthreads) {
  if (rows < 0 || d <= 0) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
  for (int64_t r = 0; r < rows; ++r) {
    const double *yr = y + r * d;
    const double *zr = z + r * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += yr[i] * yr[i];
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) {
      const double gate = 1.0 / (1.0 + exp(-zr[i]));
      const double gain = 1.0 + (w ? w[i] : 0.0);
      o[r * d + i] = gate * yr[i] * inv * gain;
    }
  }
  return 0;
}

/* Gradients of L = <dy, y> + <dS_T, S_T> with respect to q, k, v,
 * log_alpha, beta and S0 (dS_T and S0 may be NULL: zeros). Layouts as the
 * forward; the outputs dq, dk, dv, dlog_alpha, dbeta, dS0 have the shapes of
 * q, k, v, log_alpha, beta and S0 ([N, H, dk, dv]). Every state S_t of a
 * (sequence, head) is kept in memory for the backward sweep. */
int oracle_gdn_bwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta,
                   const double *S0, const double *dy, const double *dS_T,
                   const int32_t *cu_seqlens, int N, int T, int H, int dk,
                   int dv, double *dq, double *dk_out, double *dv_out,
                   double *dlog_alpha, double *dbeta, double *dS0,
                   int nthreads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const size_t state = (size_t)dk * dv;
  const int64_t units = (int64_t)N * H;
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t nh = 0; nh < units; ++nh) {
    const int h = (int)(nh % H);
    const int n = (int)(nh / H);
    const int64_t t0 = seq_start(cu_seqlens, n, T);
    const int64_t len = seq_len(cu_seqlens, n, T);
    double *hist = (double *)malloc(sizeof(double) * state * (size_t)(len + 1));
    double *dS = (double *)malloc(sizeof(double) * state);
    double *St = (double *)malloc(sizeof(double) * state);
    double *e = (double *)malloc(sizeof(double) * (size_t)dv);
    double *de = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!hist || !dS || !St || !e || !de) {
      free(hist); free(dS); free(St); free(e); free(de);
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = -2;
      continue;
    }
    /* forward sweep: hist[t] = S_t (S_0 = the initial state) */
    if (S0) memcpy(hist, S0 + nh * state, sizeof(double) * state);
    else memset(hist, 0, sizeof(double) * state);
    for (int64_t t = 0; t < len; ++t) {
      const int64_t row = (t0 + t) * H + h;
      const double a = exp(log_alpha[row]);
      const double b = beta[row];
      const double *kt = k + row * dk;
      const double *vt = v + row * dv;
      const double *Sp = hist + (size_t)t * state;
      double *Sn = hist + (size_t)(t + 1) * state;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += a * Sp[i * dv + j] * kt[i];
        e[j] = vt[j] - acc;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) Sn[i * dv + j] = a * Sp[i * dv + j] + b * kt[i] * e[j];
    }
    /* backward sweep */
    if (dS_T) memcpy(dS, dS_T + nh * state, sizeof(double) * state);
    else memset(dS, 0, sizeof(double) * state);
    for (int64_t t = len - 1; t >= 0; --t) {
      const int64_t row = (t0 + t) * H + h;
      const double a = exp(log_alpha[row]);
      const double b = beta[row];
      const double *qt = q + row * dk;
      const double *kt = k + row * dk;
      const double *vt = v + row * dv;
      const double *dyt = dy + row * dv;
      const double *Sp = hist + (size_t)t * state;
      const double *Sn = hist + (size_t)(t + 1) * state;
      /* recompute the error against the decayed state */
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += a * Sp[i * dv + j] * kt[i];
        e[j] = vt[j] - acc;
      }
      /* y_t = S_t^T q_t */
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += Sn[i * dv + j] * dyt[j];
        dq[row * dk + i] = acc;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) dS[i * dv + j] += qt[i] * dyt[j];
      /* S_t = S~ + beta k e^T */
      double db = 0.0;
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += dS[i * dv + j] * e[j];
        db += kt[i] * acc;
        dk_out[row * dk + i] = b * acc; /* the S~ de part follows below */
      }
      dbeta[row] = db;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += dS[i * dv + j] * kt[i];
        de[j] = b * acc;
        dv_out[row * dv + j] = de[j];
      }
      /* e = v - S~^T k */
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += a * Sp[i * dv + j] * de[j];
        dk_out[row * dk + i] -= acc;
      }
      /* S~ = alpha S_{t-1} */
      double dalpha = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
          const double dSt = dS[i * dv + j] - kt[i] * de[j];
          dalpha += Sp[i * dv + j] * dSt;
          dS[i * dv + j] = a * dSt;
        }
      dlog_alpha[row] = a * dalpha;
    }
    memcpy(dS0 + nh * state, dS, sizeof(double) * state);
    free(hist); free(dS); free(St); free(e); free(de);
  }
  return status;
}

/* Gates from raw pre-activations a, b [rows, H] with per-head A [H] and
 * b_alpha [H] (may be NULL: zero):
 *   log_alpha = -exp(A_h) * softplus(a + b_alpha_h),  beta = 1 / (1 + exp(-b)),
 * softplus(x) = log(1 + exp(x)) evaluated as max(x, 0) + log1p(exp(-|x|)). */
int oracle_gates_from_raw(const double *a, const double *b, const double *A,
                          const double *b_alpha, double *log_alpha,
                          double *beta, int64_t rows, int H) {
  if (rows < 0 || H <= 0) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int h = 0; h < H; ++h) {
      const int64_t i = r * H + h;
      const double x = a[i] + (b_alpha ? b_alpha[h] : 0.0);
      const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
      log_alpha[i] = -exp(A[h]) * sp;
      beta[i] = 1.0 / (1.0 + exp(-b[i]));
    }
  }
  return 0;
}

/* Gradients through the gate map above: given dlog_alpha and dbeta [rows,
 * H], returns da, db [rows, H] and the per-head sums dA, db_alpha [H]:
 *   d a       = dlog_alpha * (-exp(A_h) * sigmoid(a + b_alpha_h))
 *   d b       = dbeta * beta (1 - beta),   beta = sigmoid(b)
 *   d A_h     = sum over rows of dlog_alpha * log_alpha
 *   d b_alpha = sum over rows of d a. */
int oracle_gates_from_raw_bwd(const double *a, const double *b, const double *A,
                              const double *b_alpha, const double *dlog_alpha,
                              const double *dbeta, double *da, double *db,
                              double *dA, double *db_alpha, int64_t rows, int H) {
  if (rows < 0 || H <= 0) return -1;
  for (int h = 0; h < H; ++h) {
    dA[h] = 0.0;
    db_alpha[h] = 0.0;
  }
  for (int64_t r = 0; r < rows; ++r) {
    for (int h = 0; h < H; ++h) {
      const int64_t i = r * H + h;
      const double x = a[i] + (b_alpha ? b_alpha[h] : 0.0);
      const double sig = 1.0 / (1.0 + exp(-x));
      const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
      const double la = -exp(A[h]) * sp;
      da[i] = dlog_alpha[i] * (-exp(A[h]) * sig);
      const double bt = 1.0 / (1.0 + exp(-b[i]));
      db[i] = dbeta[i] * bt * (1.0 - bt);
      dA[h] += dlog_alpha[i] * la;
      db_alpha[h] += da[i];
    }
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

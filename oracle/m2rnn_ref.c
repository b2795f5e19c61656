/*
 * m2rnn_ref.c -- plain, slow, obviously-correct fp64 oracle of the M2RNN scan.
 *
 * TEST INFRASTRUCTURE ONLY (see m2rnn_ref.h).  Every loop below is the plain
 * definition; there is no blocking, fusion or reordering beyond the order in
 * which the equations are written on the slides.
 *
 * Forward, per (batch b, value head n), slide "Write, transform, retain, and
 * read a matrix state" (paper Eqs. (10)-(12)), with H_0 = 0 as the slides fix
 * it, or a caller-given H_0 (the same recurrence resumed from a stored state,
 * so that a sequence can be split across calls):
 *     Z_t = tanh(H_{t-1} W + k_t v_t^T)
 *     H_t = f_t H_{t-1} + (1 - f_t) Z_t
 *     y_t = H_t^T q_t + w_r (.) v_t
 * q_t and k_t are shared by the N value heads of a token, slide "Shared
 * queries and keys buy more recurrent capacity" (paper Alg. 1).
 *
 * Backward, slide "Backup: the recurrent gradient needs both paths": with
 * u_t = dL/dy_t and C_t the gradient reaching H_t from later steps,
 *     R_t     = C_t + q_t u_t^T
 *     D_t     = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t)
 *     C_{t-1} = f_t R_t + D_t W^T
 *     dL/df_t = <R_t, H_{t-1} - Z_t>_F
 *     dL/dW   = sum_t H_{t-1}^T D_t
 * The slide leaves the value-residual and input gradients to the reader; the
 * plain chain rule on the forward equations gives
 *     dL/dk_t = D_t v_t,            dL/dv_t = D_t^T k_t + w_r (.) u_t,
 *     dL/dq_t = H_t u_t,            dL/dw_r = sum_t u_t (.) v_t,
 * with dq, dk summed over the heads that share q_t, k_t.  The recursion for C
 * ends at C_0 = dL/dH_0, the gradient of a caller-given initial state.
 */
#include "m2rnn_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
  int B, T, N, K, V;
  const double *q, *k, *v, *f, *W, *wr;
  const double* H_0; /* NULL: zero initial state */
  /* forward outputs */
  double *y, *H_T, *H_ckpt;
  int ckpt_every;
  /* backward inputs / outputs */
  const double *dy, *dH_T;
  double *dv, *df;
  double* dH_0;             /* NULL: not wanted */
  double *dq_part, *dk_part; /* [B][N][T][K] per-chain contributions */
  double *dW_part, *dwr_part; /* [B][N][V][V], [B][N][V] */
  int nthreads, tid;
  int status;
} job_t;

static int resolve_threads(int nthreads, int chains) {
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > chains) nthreads = chains;
  if (nthreads < 1) nthreads = 1;
  return nthreads;
}

/* One step of the recurrence for chain (b, n) at time t: Hn = new state,
 * Z = candidate, from Hp = previous state.  Returns nothing; pure function of
 * its arguments. */
static void step(const job_t* J, int b, int n, int t, const double* Hp,
                 double* A, double* Z, double* Hn) {
  const int K = J->K, V = J->V, N = J->N, T = J->T;
  const double* kt = J->k + ((size_t)b * T + t) * K;
  const double* vt = J->v + (((size_t)b * T + t) * N + n) * V;
  const double ft = J->f[((size_t)b * T + t) * N + n];
  const double* Wn = J->W + (size_t)n * V * V;
  /* A = H_{t-1} W + k_t v_t^T */
  for (int i = 0; i < K; ++i) {
    for (int j = 0; j < V; ++j) {
      double s = 0.0;
      for (int l = 0; l < V; ++l) s += Hp[i * V + l] * Wn[l * V + j];
      A[i * V + j] = s + kt[i] * vt[j];
    }
  }
  /* Z = tanh(A);  H_t = f H_{t-1} + (1 - f) Z */
  for (int e = 0; e < K * V; ++e) {
    Z[e] = tanh(A[e]);
    Hn[e] = ft * Hp[e] + (1.0 - ft) * Z[e];
  }
}

/* y_t = H_t^T q_t + w_r (.) v_t for chain (b, n). */
static void readout(const job_t* J, int b, int n, int t, const double* H) {
  const int K = J->K, V = J->V, N = J->N, T = J->T;
  const double* qt = J->q + ((size_t)b * T + t) * K;
  const double* vt = J->v + (((size_t)b * T + t) * N + n) * V;
  const double* wrn = J->wr + (size_t)n * V;
  double* yt = J->y + (((size_t)b * T + t) * N + n) * V;
  for (int j = 0; j < V; ++j) {
    double s = 0.0;
    for (int i = 0; i < K; ++i) s += H[i * V + j] * qt[i];
    yt[j] = s + wrn[j] * vt[j];
  }
}

static void* forward_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int K = J->K, V = J->V, N = J->N, T = J->T;
  const size_t S = (size_t)K * V;
  double* buf = (double*)malloc(sizeof(double) * 4 * S);
  if (!buf) { J->status = -2; return NULL; }
  double *H = buf, *A = buf + S, *Z = buf + 2 * S, *Hn = buf + 3 * S;
  const int nck = J->ckpt_every > 0 ? (T + J->ckpt_every - 1) / J->ckpt_every : 0;
  for (int c = J->tid; c < J->B * N; c += J->nthreads) {
    const int b = c / N, n = c % N;
    if (J->H_0) memcpy(H, J->H_0 + ((size_t)b * N + n) * S, sizeof(double) * S);
    else memset(H, 0, sizeof(double) * S); /* H_0 = 0 */
    for (int t = 0; t < T; ++t) {
      if (J->H_ckpt && J->ckpt_every > 0 && t % J->ckpt_every == 0) {
        double* dst = J->H_ckpt + (((size_t)b * N + n) * nck + t / J->ckpt_every) * S;
        memcpy(dst, H, sizeof(double) * S);
      }
      step(J, b, n, t, H, A, Z, Hn);
      memcpy(H, Hn, sizeof(double) * S);
      readout(J, b, n, t, H);
    }
    memcpy(J->H_T + ((size_t)b * N + n) * S, H, sizeof(double) * S);
  }
  free(buf);
  return NULL;
}

static void* backward_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int K = J->K, V = J->V, N = J->N, T = J->T;
  const size_t S = (size_t)K * V;
  /* Hs[t] = H_t for t = 0..T, Zs[t] = Z_{t+1} for t = 0..T-1 */
  double* Hs = (double*)malloc(sizeof(double) * (size_t)(T + 1) * S);
  double* Zs = (double*)malloc(sizeof(double) * (size_t)T * S);
  double* work = (double*)malloc(sizeof(double) * 4 * S);
  if (!Hs || !Zs || !work) {
    free(Hs); free(Zs); free(work);
    J->status = -2;
    return NULL;
  }
  double *A = work, *C = work + S, *R = work + 2 * S, *D = work + 3 * S;
  for (int c = J->tid; c < J->B * N; c += J->nthreads) {
    const int b = c / N, n = c % N;
    const double* Wn = J->W + (size_t)n * V * V;
    const double* wrn = J->wr + (size_t)n * V;
    double* dWc = J->dW_part + ((size_t)b * N + n) * V * V;
    double* dwrc = J->dwr_part + ((size_t)b * N + n) * V;
    memset(dWc, 0, sizeof(double) * V * V);
    memset(dwrc, 0, sizeof(double) * V);

    /* recompute and keep the whole trajectory */
    if (J->H_0) memcpy(Hs, J->H_0 + ((size_t)b * N + n) * S, sizeof(double) * S);
    else memset(Hs, 0, sizeof(double) * S);
    for (int t = 0; t < T; ++t) step(J, b, n, t, Hs + (size_t)t * S, A, Zs + (size_t)t * S, Hs + (size_t)(t + 1) * S);

    /* C_T = dL/dH_T (only the final-state term) */
    if (J->dH_T) memcpy(C, J->dH_T + ((size_t)b * N + n) * S, sizeof(double) * S);
    else memset(C, 0, sizeof(double) * S);

    for (int t = T - 1; t >= 0; --t) {
      const double* Hp = Hs + (size_t)t * S;       /* H_{t-1} in 1-based notation */
      const double* Hc = Hs + (size_t)(t + 1) * S; /* H_t */
      const double* Z = Zs + (size_t)t * S;        /* Z_t */
      const double* qt = J->q + ((size_t)b * T + t) * K;
      const double* kt = J->k + ((size_t)b * T + t) * K;
      const double* vt = J->v + (((size_t)b * T + t) * N + n) * V;
      const double ft = J->f[((size_t)b * T + t) * N + n];
      const double* u = J->dy + (((size_t)b * T + t) * N + n) * V;

      /* R_t = C_t + q_t u_t^T;  D_t = ((1 - f) R_t) (.) (1 - Z (.) Z) */
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) R[i * V + j] = C[i * V + j] + qt[i] * u[j];
      for (int e = 0; e < (int)S; ++e) D[e] = ((1.0 - ft) * R[e]) * (1.0 - Z[e] * Z[e]);

      /* dL/df_t = <R_t, H_{t-1} - Z_t> */
      double s = 0.0;
      for (int e = 0; e < (int)S; ++e) s += R[e] * (Hp[e] - Z[e]);
      J->df[((size_t)b * T + t) * N + n] = s;

      /* dL/dW += H_{t-1}^T D_t */
      for (int l = 0; l < V; ++l)
        for (int j = 0; j < V; ++j) {
          double a = 0.0;
          for (int i = 0; i < K; ++i) a += Hp[i * V + l] * D[i * V + j];
          dWc[l * V + j] += a;
        }

      /* dL/dk_t (this head's share) = D_t v_t */
      double* dkp = J->dk_part + (((size_t)b * N + n) * T + t) * K;
      for (int i = 0; i < K; ++i) {
        double a = 0.0;
        for (int j = 0; j < V; ++j) a += D[i * V + j] * vt[j];
        dkp[i] = a;
      }
      /* dL/dv_t = D_t^T k_t + w_r (.) u_t */
      double* dvt = J->dv + (((size_t)b * T + t) * N + n) * V;
      for (int j = 0; j < V; ++j) {
        double a = 0.0;
        for (int i = 0; i < K; ++i) a += D[i * V + j] * kt[i];
        dvt[j] = a + wrn[j] * u[j];
      }
      /* dL/dq_t (this head's share) = H_t u_t */
      double* dqp = J->dq_part + (((size_t)b * N + n) * T + t) * K;
      for (int i = 0; i < K; ++i) {
        double a = 0.0;
        for (int j = 0; j < V; ++j) a += Hc[i * V + j] * u[j];
        dqp[i] = a;
      }
      /* dL/dw_r += u_t (.) v_t */
      for (int j = 0; j < V; ++j) dwrc[j] += u[j] * vt[j];

      /* C_{t-1} = f R_t + D_t W^T,  (D W^T)[i][l] = sum_j D[i][j] W[l][j] */
      for (int i = 0; i < K; ++i)
        for (int l = 0; l < V; ++l) {
          double a = 0.0;
          for (int j = 0; j < V; ++j) a += D[i * V + j] * Wn[l * V + j];
          C[i * V + l] = ft * R[i * V + l] + a;
        }
    }
    /* C_0 = dL/dH_0 */
    if (J->dH_0) memcpy(J->dH_0 + ((size_t)b * N + n) * S, C, sizeof(double) * S);
  }
  free(Hs); free(Zs); free(work);
  return NULL;
}

static int run_pool(job_t* base, int nthreads, void* (*fn)(void*)) {
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * nthreads);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  if (!jobs || !th) { free(jobs); free(th); return -2; }
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = *base;
    jobs[i].nthreads = nthreads;
    jobs[i].tid = i;
    jobs[i].status = 0;
  }
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, fn, &jobs[i]) != 0) break;
    started = i;
  }
  /* threads that failed to start: run their share inline afterwards */
  fn(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  for (int i = started + 1; i < nthreads; ++i) fn(&jobs[i]);
  int st = 0;
  for (int i = 0; i < nthreads; ++i) if (jobs[i].status) st = jobs[i].status;
  free(jobs); free(th);
  return st;
}

static int bad_dims(int B, int T, int N, int K, int V) {
  return B < 1 || T < 1 || N < 1 || K < 1 || V < 1;
}

int m2rnn_ref_forward(int B, int T, int N, int K, int V,
                      const double* q, const double* k, const double* v,
                      const double* f, const double* W, const double* wr,
                      const double* H_0,
                      double* y, double* H_T, double* H_ckpt, int ckpt_every,
                      int nthreads) {
  if (bad_dims(B, T, N, K, V) || !q || !k || !v || !f || !W || !wr || !y || !H_T) return -1;
  if (H_ckpt && ckpt_every < 1) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.B = B; J.T = T; J.N = N; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.f = f; J.W = W; J.wr = wr; J.H_0 = H_0;
  J.y = y; J.H_T = H_T; J.H_ckpt = H_ckpt; J.ckpt_every = ckpt_every;
  return run_pool(&J, resolve_threads(nthreads, B * N), forward_worker);
}

int m2rnn_ref_backward(int B, int T, int N, int K, int V,
                       const double* q, const double* k, const double* v,
                       const double* f, const double* W, const double* wr,
                       const double* H_0,
                       const double* dy, const double* dH_T,
                       double* dq, double* dk, double* dv, double* df,
                       double* dW, double* dwr, double* dH_0, int nthreads) {
  if (bad_dims(B, T, N, K, V) || !q || !k || !v || !f || !W || !wr || !dy ||
      !dq || !dk || !dv || !df || !dW || !dwr) return -1;
  const size_t part = (size_t)B * N * T * K;
  job_t J;
  memset(&J, 0, sizeof J);
  J.B = B; J.T = T; J.N = N; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.f = f; J.W = W; J.wr = wr; J.H_0 = H_0;
  J.dy = dy; J.dH_T = dH_T; J.dv = dv; J.df = df; J.dH_0 = dH_0;
  J.dq_part = (double*)malloc(sizeof(double) * part);
  J.dk_part = (double*)malloc(sizeof(double) * part);
  J.dW_part = (double*)malloc(sizeof(double) * (size_t)B * N * V * V);
  J.dwr_part = (double*)malloc(sizeof(double) * (size_t)B * N * V);
  int st = -2;
  if (J.dq_part && J.dk_part && J.dW_part && J.dwr_part)
    st = run_pool(&J, resolve_threads(nthreads, B * N), backward_worker);
  if (st == 0) {
    /* shared q_t, k_t: sum the heads' contributions in ascending n */
    for (int b = 0; b < B; ++b)
      for (int t = 0; t < T; ++t)
        for (int i = 0; i < K; ++i) {
          double sq = 0.0, sk = 0.0;
          for (int n = 0; n < N; ++n) {
            sq += J.dq_part[(((size_t)b * N + n) * T + t) * K + i];
            sk += J.dk_part[(((size_t)b * N + n) * T + t) * K + i];
          }
          dq[((size_t)b * T + t) * K + i] = sq;
          dk[((size_t)b * T + t) * K + i] = sk;
        }
    /* W and w_r are shared by every batch row: sum in ascending b */
    for (int n = 0; n < N; ++n) {
      for (int e = 0; e < V * V; ++e) {
        double s = 0.0;
        for (int b = 0; b < B; ++b) s += J.dW_part[((size_t)b * N + n) * V * V + e];
        dW[(size_t)n * V * V + e] = s;
      }
      for (int j = 0; j < V; ++j) {
        double s = 0.0;
        for (int b = 0; b < B; ++b) s += J.dwr_part[((size_t)b * N + n) * V + j];
        dwr[(size_t)n * V + j] = s;
      }
    }
  }
  free(J.dq_part); free(J.dk_part); free(J.dW_part); free(J.dwr_part);
  return st;
}

/* ------------------------------------------------------------------ gate
 * Forget gate from a pre-activation, slide "The gate preserves a direct path
 * through time" (paper Sec. 3.1, Eqs. (13), (17)):
 *     f[b][t][n] = exp(-alpha[n] * softplus(a[b][t][n] + beta[n])),
 * softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(exp(-|x|)).
 * Backward, by the chain rule with softplus'(x) = 1 / (1 + e^{-x}):
 *     da    = df * f * (-alpha) * sigmoid(a + beta)
 *     dalpha = sum_{b,t} df * f * (-softplus(a + beta))
 *     dbeta  = sum_{b,t} da
 * (sums over b ascending, then t ascending). */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

int m2rnn_ref_gate_forward(int B, int T, int N, const double* a, const double* alpha, const double* beta,
                           double* f) {
  if (B < 0 || T < 0 || N < 1 || !a || !alpha || !beta || !f) return -1;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int n = 0; n < N; ++n) {
        const size_t i = ((size_t)b * T + t) * N + n;
        f[i] = exp(-alpha[n] * softplus(a[i] + beta[n]));
      }
  return 0;
}

int m2rnn_ref_gate_backward(int B, int T, int N, const double* a, const double* alpha, const double* beta,
                            const double* df, double* da, double* dalpha, double* dbeta) {
  if (B < 0 || T < 0 || N < 1 || !a || !alpha || !beta || !df || !da || !dalpha || !dbeta) return -1;
  for (int n = 0; n < N; ++n) { dalpha[n] = 0.0; dbeta[n] = 0.0; }
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int n = 0; n < N; ++n) {
        const size_t i = ((size_t)b * T + t) * N + n;
        const double x = a[i] + beta[n];
        const double sp = softplus(x);
        const double f = exp(-alpha[n] * sp);
        const double sig = 1.0 / (1.0 + exp(-x));
        da[i] = df[i] * f * (-alpha[n]) * sig;
        dalpha[n] += df[i] * f * (-sp);
        dbeta[n] += da[i];
      }
  return 0;
}

/* ---------------------------------------------------- output gate, RMSNorm
 * After the readout the block multiplies by the output gate g and applies
 * RMSNorm over the token's d = N V features (slide "Most of the block can be
 * computed before recurrence", paper Fig. 2), with the statistic of slide
 * "Backup: RMSNormTP synchronizes per-token statistics" (paper App. C, Eqs.
 * (26)-(33)), here over one device's whole feature vector:
 *     x = y (.) g,   s = [ (1/d) sum_j x_j^2 + eps ]^{-1/2},   o_i = w_i x_i s
 * (the pages omit eps; eps = 0 is their form).  Backward, as on that slide:
 *     p_i = w_i do_i,   r = sum_j p_j x_j,   dx_i = s p_i - r s^3 x_i / d
 * and by the chain rule through x = y (.) g and o = w (.) (x s):
 *     dy = dx (.) g,   dg = dx (.) y,   dw_i = sum over tokens of do_i x_i s
 * (tokens in ascending order).  One token is a row of d values. */
int m2rnn_ref_gate_rmsnorm_forward(int ntok, int d, const double* y, const double* g, const double* w,
                                   double eps, double* o, double* rstd) {
  if (ntok < 0 || d < 1 || eps < 0.0 || !y || !g || !w || !o) return -1;
  for (int t = 0; t < ntok; ++t) {
    const double* yt = y + (size_t)t * d;
    const double* gt = g + (size_t)t * d;
    double ss = 0.0;
    for (int j = 0; j < d; ++j) ss += (yt[j] * gt[j]) * (yt[j] * gt[j]);
    const double s = 1.0 / sqrt(ss / d + eps);
    for (int j = 0; j < d; ++j) o[(size_t)t * d + j] = w[j] * (yt[j] * gt[j]) * s;
    if (rstd) rstd[t] = s;
  }
  return 0;
}

int m2rnn_ref_gate_rmsnorm_backward(int ntok, int d, const double* y, const double* g, const double* w,
                                    double eps, const double* dout, double* dy, double* dg, double* dw) {
  if (ntok < 0 || d < 1 || eps < 0.0 || !y || !g || !w || !dout || !dy || !dg || !dw) return -1;
  double* x = (double*)malloc(sizeof(double) * d);
  if (!x) return -2;
  for (int j = 0; j < d; ++j) dw[j] = 0.0;
  for (int t = 0; t < ntok; ++t) {
    const double* yt = y + (size_t)t * d;
    const double* gt = g + (size_t)t * d;
    const double* dt = dout + (size_t)t * d;
    double ss = 0.0;
    for (int j = 0; j < d; ++j) {
      x[j] = yt[j] * gt[j];
      ss += x[j] * x[j];
    }
    const double s = 1.0 / sqrt(ss / d + eps);
    double r = 0.0;
    for (int j = 0; j < d; ++j) r += (w[j] * dt[j]) * x[j];
    for (int j = 0; j < d; ++j) {
      const double dx = s * (w[j] * dt[j]) - r * s * s * s * x[j] / d;
      dy[(size_t)t * d + j] = dx * gt[j];
      dg[(size_t)t * d + j] = dx * yt[j];
      dw[j] += dt[j] * x[j] * s;
    }
  }
  free(x);
  return 0;
}

/* -------------------------------------------------- causal Conv1D and SiLU
 * Before the scan, q, k and v come out of a linear projection, a causal
 * Conv1D of width 4 and a SiLU (slide "Most of the block can be computed
 * before recurrence", paper Fig. 2).  Read as a depthwise convolution over
 * time per channel c, with zero input before t = 0 and an optional bias,
 * taps in the order of a cross-correlation (the last tap on the current step):
 *     a[b][t][c] = bias[c] + sum_{j=0..3} w[c][j] u[b][t-3+j][c]
 *     z = silu(a) = a / (1 + e^{-a})
 * Backward from dz, with silu'(a) = s (1 + a (1 - s)), s = 1 / (1 + e^{-a}):
 *     da = dz silu'(a)
 *     du[b][t][c] = sum_j w[c][j] da[b][t+3-j][c]   (terms past T are zero)
 *     dw[c][j] = sum_{b,t} da[b][t][c] u[b][t-3+j][c],   dbias[c] = sum_{b,t} da
 * (sums over b ascending, then t ascending). */
#define CONV_W 4

static double conv_pre(int T, int C, const double* u, const double* w, const double* bias, int b, int t, int c) {
  double a = bias ? bias[c] : 0.0;
  for (int j = 0; j < CONV_W; ++j) {
    const int ts = t - (CONV_W - 1) + j;
    if (ts >= 0) a += w[c * CONV_W + j] * u[((size_t)b * T + ts) * C + c];
  }
  return a;
}

int m2rnn_ref_conv_silu_forward(int B, int T, int C, const double* u, const double* w, const double* bias,
                                double* z) {
  if (B < 0 || T < 0 || C < 1 || !u || !w || !z) return -1;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int c = 0; c < C; ++c) {
        const double a = conv_pre(T, C, u, w, bias, b, t, c);
        z[((size_t)b * T + t) * C + c] = a / (1.0 + exp(-a));
      }
  return 0;
}

int m2rnn_ref_conv_silu_backward(int B, int T, int C, const double* u, const double* w, const double* bias,
                                 const double* dz, double* du, double* dw, double* dbias) {
  if (B < 0 || T < 0 || C < 1 || !u || !w || !dz || !du || !dw) return -1;
  double* da = (double*)malloc(sizeof(double) * ((size_t)T > 0 ? (size_t)T : 1));
  if (!da) return -2;
  for (int e = 0; e < C * CONV_W; ++e) dw[e] = 0.0;
  if (dbias)
    for (int c = 0; c < C; ++c) dbias[c] = 0.0;
  for (int c = 0; c < C; ++c)
    for (int b = 0; b < B; ++b) {
      for (int t = 0; t < T; ++t) {
        const double a = conv_pre(T, C, u, w, bias, b, t, c);
        const double s = 1.0 / (1.0 + exp(-a));
        da[t] = dz[((size_t)b * T + t) * C + c] * s * (1.0 + a * (1.0 - s));
      }
      for (int t = 0; t < T; ++t) {
        double g = 0.0;
        for (int j = 0; j < CONV_W; ++j) {
          const int to = t + (CONV_W - 1) - j;
          if (to < T) g += w[c * CONV_W + j] * da[to];
        }
        du[((size_t)b * T + t) * C + c] = g;
        for (int j = 0; j < CONV_W; ++j) {
          const int ts = t - (CONV_W - 1) + j;
          if (ts >= 0) dw[c * CONV_W + j] += da[t] * u[((size_t)b * T + ts) * C + c];
        }
        if (dbias) dbias[c] += da[t];
      }
    }
  free(da);
  return 0;
}

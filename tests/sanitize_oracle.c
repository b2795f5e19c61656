/*
 * Memory- and UB-safety driver for the fp64 CPU oracle (oracle/m2rnn_ref.c),
 * built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py.  Every entry point runs on odd sizes
 * (K, V not multiples of anything the GPU path uses, T shorter and longer
 * than the checkpoint interval), with and without each optional argument,
 * on one, several and all host threads, and with bad arguments; every
 * buffer is its own exact-size heap block, so a read or write one element
 * past any tensor is reported.  A few invariants are checked on the way:
 * the checkpoints are the states a run from H_0 passes through, a run
 * restarted from a checkpoint ends in the same H_T, and results are finite.
 * Exit status 0 means every call behaved; the sanitizers abort on the first
 * fault.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "m2rnn_ref.h"

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;

/* uniform in [-s, s) from a 64-bit linear congruential generator */
static double urand(double s) {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return s * (2.0 * (double)(rng_state >> 11) / 9007199254740992.0 - 1.0);
}

static double* alloc(size_t n) {
  double* p = (double*)malloc((n ? n : 1) * sizeof(double));
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static double* rnd(size_t n, double s) {
  double* p = alloc(n);
  for (size_t i = 0; i < n; ++i) p[i] = urand(s);
  return p;
}

static double* gate(size_t n) {  /* forget gates in [0.05, 0.95] */
  double* p = alloc(n);
  for (size_t i = 0; i < n; ++i) p[i] = 0.5 + urand(0.45);
  return p;
}

static int failures = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static double max_abs_diff(const double* a, const double* b, size_t n) {
  double m = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double d = fabs(a[i] - b[i]);
    if (d > m) m = d;
  }
  return m;
}

/* one forward + backward configuration */
static void scan_case(int B, int T, int N, int K, int V, int ck, int with_h0, int with_dht, int with_dh0,
                      int nthreads) {
  const size_t nqk = (size_t)B * T * K, nv = (size_t)B * T * N * V, nf = (size_t)B * T * N;
  const size_t nH = (size_t)B * N * K * V, nck = (size_t)(T + ck - 1) / ck;
  double *q = rnd(nqk, 1.0), *k = rnd(nqk, 1.0), *v = rnd(nv, 1.0), *f = gate(nf);
  double *W = rnd((size_t)N * V * V, 0.25), *wr = rnd((size_t)N * V, 0.5);
  double* H0 = with_h0 ? rnd(nH, 0.5) : NULL;
  double *y = alloc(nv), *HT = alloc(nH), *Hck = alloc((size_t)B * N * nck * K * V);
  char what[160];
  snprintf(what, sizeof what, "forward B=%d T=%d N=%d K=%d V=%d ckpt=%d h0=%d threads=%d", B, T, N, K, V, ck,
           with_h0, nthreads);
  check(m2rnn_ref_forward(B, T, N, K, V, q, k, v, f, W, wr, H0, y, HT, Hck, ck, nthreads) == 0, what);
  check(finite_all(y, nv) && finite_all(HT, nH), what);
  /* without checkpoints: the same y and H_T */
  {
    double *y2 = alloc(nv), *HT2 = alloc(nH);
    check(m2rnn_ref_forward(B, T, N, K, V, q, k, v, f, W, wr, H0, y2, HT2, NULL, ck, 1) == 0, what);
    check(max_abs_diff(y, y2, nv) == 0.0 && max_abs_diff(HT, HT2, nH) == 0.0, "forward without checkpoints");
    free(y2);
    free(HT2);
  }
  /* checkpoint 0 is H_0; a run restarted from the last checkpoint ends in H_T */
  {
    const int j = (int)nck - 1, t0 = j * ck, T2 = T - t0;
    double* start = alloc(nH);
    for (int b = 0; b < B; ++b)
      for (int n = 0; n < N; ++n) {
        const double* src = Hck + (((size_t)b * N + n) * nck + j) * K * V;
        memcpy(start + ((size_t)b * N + n) * K * V, src, (size_t)K * V * sizeof(double));
        const double* c0 = Hck + (((size_t)b * N + n) * nck) * K * V;
        for (int e = 0; e < K * V; ++e)
          check(c0[e] == (H0 ? H0[((size_t)b * N + n) * K * V + e] : 0.0), "checkpoint 0 is H_0");
      }
    double *q2 = alloc((size_t)B * T2 * K), *k2 = alloc((size_t)B * T2 * K), *v2 = alloc((size_t)B * T2 * N * V);
    double *f2 = alloc((size_t)B * T2 * N), *y2 = alloc((size_t)B * T2 * N * V), *HT2 = alloc(nH);
    for (int b = 0; b < B; ++b) {
      memcpy(q2 + (size_t)b * T2 * K, q + ((size_t)b * T + t0) * K, (size_t)T2 * K * sizeof(double));
      memcpy(k2 + (size_t)b * T2 * K, k + ((size_t)b * T + t0) * K, (size_t)T2 * K * sizeof(double));
      memcpy(v2 + (size_t)b * T2 * N * V, v + ((size_t)b * T + t0) * N * V, (size_t)T2 * N * V * sizeof(double));
      memcpy(f2 + (size_t)b * T2 * N, f + ((size_t)b * T + t0) * N, (size_t)T2 * N * sizeof(double));
    }
    check(m2rnn_ref_forward(B, T2, N, K, V, q2, k2, v2, f2, W, wr, start, y2, HT2, NULL, ck, 2) == 0, what);
    check(max_abs_diff(HT, HT2, nH) <= 1e-12, "restart from the last checkpoint ends in H_T");
    free(start);
    free(q2);
    free(k2);
    free(v2);
    free(f2);
    free(y2);
    free(HT2);
  }
  /* backward */
  {
    double *dy = rnd(nv, 1.0), *dHT = with_dht ? rnd(nH, 1.0) : NULL;
    double *dq = alloc(nqk), *dk = alloc(nqk), *dv = alloc(nv), *df = alloc(nf);
    double *dW = alloc((size_t)N * V * V), *dwr = alloc((size_t)N * V), *dH0 = with_dh0 ? alloc(nH) : NULL;
    snprintf(what, sizeof what, "backward B=%d T=%d N=%d K=%d V=%d h0=%d dHT=%d dH0=%d threads=%d", B, T, N, K, V,
             with_h0, with_dht, with_dh0, nthreads);
    check(m2rnn_ref_backward(B, T, N, K, V, q, k, v, f, W, wr, H0, dy, dHT, dq, dk, dv, df, dW, dwr, dH0,
                             nthreads) == 0,
          what);
    check(finite_all(dq, nqk) && finite_all(dk, nqk) && finite_all(dv, nv) && finite_all(df, nf) &&
              finite_all(dW, (size_t)N * V * V) && finite_all(dwr, (size_t)N * V) && (!dH0 || finite_all(dH0, nH)),
          what);
    free(dy);
    free(dHT);
    free(dq);
    free(dk);
    free(dv);
    free(df);
    free(dW);
    free(dwr);
    free(dH0);
  }
  free(q);
  free(k);
  free(v);
  free(f);
  free(W);
  free(wr);
  free(H0);
  free(y);
  free(HT);
  free(Hck);
}

static void bad_arguments(void) {
  double x[64] = {0}, y[64];
  check(m2rnn_ref_forward(0, 1, 1, 1, 1, x, x, x, x, x, x, NULL, y, y, NULL, 1, 1) == -1, "B = 0 rejected");
  check(m2rnn_ref_forward(1, -1, 1, 1, 1, x, x, x, x, x, x, NULL, y, y, NULL, 1, 1) == -1, "T < 0 rejected");
  check(m2rnn_ref_forward(1, 1, 1, 1, 1, NULL, x, x, x, x, x, NULL, y, y, NULL, 1, 1) == -1, "q NULL rejected");
  check(m2rnn_ref_forward(1, 1, 1, 1, 1, x, x, x, x, x, x, NULL, NULL, y, NULL, 1, 1) == -1, "y NULL rejected");
  check(m2rnn_ref_backward(1, 1, 0, 1, 1, x, x, x, x, x, x, NULL, x, NULL, y, y, y, y, y, y, NULL, 1) == -1,
        "backward N = 0 rejected");
  check(m2rnn_ref_backward(1, 1, 1, 1, 1, x, x, x, x, x, x, NULL, NULL, NULL, y, y, y, y, y, y, NULL, 1) == -1,
        "backward dy NULL rejected");
  check(m2rnn_ref_gate_forward(1, 1, 0, x, x, x, y) == -1, "gate N = 0 rejected");
  check(m2rnn_ref_gate_rmsnorm_forward(-1, 4, x, x, x, 1e-6, y, NULL) == -1, "rmsnorm ntok < 0 rejected");
  check(m2rnn_ref_gate_rmsnorm_forward(0, 4, x, x, x, 1e-6, y, NULL) == 0, "rmsnorm of no tokens is a no-op");
  check(m2rnn_ref_gate_rmsnorm_forward(1, 0, x, x, x, 1e-6, y, NULL) == -1, "rmsnorm d = 0 rejected");
  check(m2rnn_ref_conv_silu_forward(1, 1, 0, x, x, NULL, y) == -1, "conv C = 0 rejected");
}

static void gate_cases(int B, int T, int N) {
  const size_t n = (size_t)B * T * N;
  double *a = rnd(n, 3.0), *al = rnd((size_t)N, 1.0), *be = rnd((size_t)N, 1.0), *f = alloc(n);
  for (int i = 0; i < N; ++i) al[i] = fabs(al[i]) + 0.1;
  check(m2rnn_ref_gate_forward(B, T, N, a, al, be, f) == 0 && finite_all(f, n), "gate forward");
  for (size_t i = 0; i < n; ++i) check(f[i] > 0.0 && f[i] <= 1.0, "gate in (0, 1]");
  double *df = rnd(n, 1.0), *da = alloc(n), *dal = alloc((size_t)N), *dbe = alloc((size_t)N);
  check(m2rnn_ref_gate_backward(B, T, N, a, al, be, df, da, dal, dbe) == 0 && finite_all(da, n), "gate backward");
  free(a);
  free(al);
  free(be);
  free(f);
  free(df);
  free(da);
  free(dal);
  free(dbe);
}

static void norm_cases(int ntok, int d) {
  const size_t n = (size_t)ntok * d;
  double *y = rnd(n, 1.0), *g = rnd(n, 2.0), *w = rnd((size_t)d, 1.0), *o = alloc(n), *rs = alloc((size_t)ntok);
  check(m2rnn_ref_gate_rmsnorm_forward(ntok, d, y, g, w, 1e-6, o, rs) == 0 && finite_all(o, n), "rmsnorm forward");
  check(m2rnn_ref_gate_rmsnorm_forward(ntok, d, y, g, w, 1e-6, o, NULL) == 0, "rmsnorm forward without rstd");
  double *dout = rnd(n, 1.0), *dy = alloc(n), *dg = alloc(n), *dw = alloc((size_t)d);
  check(m2rnn_ref_gate_rmsnorm_backward(ntok, d, y, g, w, 1e-6, dout, dy, dg, dw) == 0 && finite_all(dy, n) &&
            finite_all(dg, n) && finite_all(dw, (size_t)d),
        "rmsnorm backward");
  free(y);
  free(g);
  free(w);
  free(o);
  free(rs);
  free(dout);
  free(dy);
  free(dg);
  free(dw);
}

static void conv_cases(int B, int T, int C) {
  const size_t n = (size_t)B * T * C;
  double *u = rnd(n, 1.0), *w = rnd((size_t)C * 4, 0.5), *bias = rnd((size_t)C, 0.1), *z = alloc(n);
  check(m2rnn_ref_conv_silu_forward(B, T, C, u, w, bias, z) == 0 && finite_all(z, n), "conv forward");
  check(m2rnn_ref_conv_silu_forward(B, T, C, u, w, NULL, z) == 0, "conv forward without bias");
  double *dz = rnd(n, 1.0), *du = alloc(n), *dw = alloc((size_t)C * 4), *db = alloc((size_t)C);
  check(m2rnn_ref_conv_silu_backward(B, T, C, u, w, bias, dz, du, dw, db) == 0 && finite_all(du, n) &&
            finite_all(dw, (size_t)C * 4) && finite_all(db, (size_t)C),
        "conv backward");
  check(m2rnn_ref_conv_silu_backward(B, T, C, u, w, NULL, dz, du, dw, NULL) == 0, "conv backward without dbias");
  free(u);
  free(w);
  free(bias);
  free(z);
  free(dz);
  free(du);
  free(dw);
  free(db);
}

int main(void) {
  /* odd sizes; checkpoint interval below, at and above T; optional arguments on and off */
  scan_case(2, 7, 3, 5, 4, 3, 1, 1, 1, 3);
  scan_case(2, 7, 3, 5, 4, 1, 0, 0, 0, 1);
  scan_case(1, 9, 2, 3, 6, 9, 1, 0, 1, 0);
  scan_case(3, 5, 1, 7, 2, 16, 0, 1, 0, 2);
  scan_case(1, 1, 1, 1, 1, 1, 1, 1, 1, 1);  /* the degenerate scalar scan */
  scan_case(1, 33, 4, 64, 16, 4, 1, 1, 1, 0);  /* the configs' K, V */
  bad_arguments();
  gate_cases(2, 5, 3);
  gate_cases(1, 1, 1);
  norm_cases(5, 7);
  norm_cases(1, 1);
  conv_cases(2, 6, 5);
  conv_cases(1, 2, 1);  /* shorter than the filter */
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: all calls clean\n");
  return 0;
}

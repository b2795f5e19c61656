/*
 * m2rnn_ref.h -- plain fp64 CPU oracle of the M2RNN matrix-state scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library: only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library (non_linear_matrix_amd/csrc) and neither side includes the other.
 *
 * Source of the method: "M2RNN: Non-Linear RNNs with Matrix-Valued States for
 * Scalable Language Modeling -- research paper discussion" (slides reading
 * Mishra, Tan, Stoica, Gonzalez, Dao, arXiv:2603.14360v2):
 *   - slide "Write, transform, retain, and read a matrix state"
 *     (paper Eqs. (10)-(12)): the recurrence;
 *   - slide "Shared queries and keys buy more recurrent capacity"
 *     (paper Alg. 1, App. A): one q/k per token shared by N value heads,
 *     one v, f, W, w_r per value head;
 *   - slide "Backup: the recurrent gradient needs both paths": the
 *     chain-rule backward for the state, f and W.
 *
 * Layouts (all dense, row-major, float64):
 *   q, k  [B][T][K]        shared by the N value heads of a batch row
 *   v     [B][T][N][V]
 *   f     [B][T][N]        scalar forget gate per (token, head)
 *   W     [N][V][V]        (H W)[i][j] = sum_l H[i][l] * W[n][l][j]
 *   wr    [N][V]           value-residual weight
 *   y     [B][T][N][V]     readout of the UPDATED state H_t
 *   H_T   [B][N][K][V]     state after the last step
 *   H_0   [B][N][K][V]     initial state; NULL means zero (the slides' H_0)
 *   H_ckpt[B][N][ceil(T/ckpt_every)][K][V]  H at t = j*ckpt_every (j = 0: H_0)
 *   dH_0  [B][N][K][V]     gradient of the initial state (backward; NULL: not
 *                          wanted)
 *
 * Any K >= 1, V >= 1 is accepted.  Return 0 on success, -1 on a bad
 * argument (null pointer, non-positive size).  nthreads <= 0 means "all
 * online CPUs".
 */
#ifndef M2RNN_REF_H
#define M2RNN_REF_H
#ifdef __cplusplus
extern "C" {
#endif

int m2rnn_ref_forward(int B, int T, int N, int K, int V,
                      const double* q, const double* k, const double* v,
                      const double* f, const double* W, const double* wr,
                      const double* H_0, /* may be NULL */
                      double* y, double* H_T,
                      double* H_ckpt, int ckpt_every, /* H_ckpt may be NULL */
                      int nthreads);

/* Gradients of L = sum(y * dy) + sum(H_T * dH_T) for the run that started
 * from H_0 (NULL: zero).  dH_T may be NULL (zero); dH_0 may be NULL.
 * dq, dk [B][T][K] are summed over the N heads (ascending n); dW [N][V][V]
 * and dwr [N][V] over batch and time (ascending b, then descending t). */
int m2rnn_ref_backward(int B, int T, int N, int K, int V,
                       const double* q, const double* k, const double* v,
                       const double* f, const double* W, const double* wr,
                       const double* H_0,
                       const double* dy, const double* dH_T,
                       double* dq, double* dk, double* dv, double* df,
                       double* dW, double* dwr, double* dH_0,
                       int nthreads);

/* Forget gate from a pre-activation (slide "The gate preserves a direct path
 * through time", paper Eqs. (13), (17)): f = exp(-alpha[n] softplus(a + beta[n]))
 * for a, f [B][T][N] and alpha, beta [N]; and its backward from df [B][T][N]:
 * da [B][T][N], dalpha and dbeta [N] summed over batch and time.  Return 0, or
 * -1 on a bad argument. */
int m2rnn_ref_gate_forward(int B, int T, int N, const double* a, const double* alpha, const double* beta,
                           double* f);
int m2rnn_ref_gate_backward(int B, int T, int N, const double* a, const double* alpha, const double* beta,
                            const double* df, double* da, double* dalpha, double* dbeta);

/* Output gate and RMSNorm after the readout (slide "Most of the block can be
 * computed before recurrence", paper Fig. 2; statistic and backward of slide
 * "Backup: RMSNormTP synchronizes per-token statistics", paper App. C, Eqs.
 * (26)-(33)): per token row of d features, x = y (.) g,
 * s = ((1/d) sum x^2 + eps)^{-1/2}, o = w (.) x s; rstd [ntok] (may be NULL)
 * receives s.  Backward from dout: dy, dg [ntok][d] and dw [d] summed over
 * tokens.  Return 0, -1 on a bad argument, -2 when out of memory. */
int m2rnn_ref_gate_rmsnorm_forward(int ntok, int d, const double* y, const double* g, const double* w,
                                   double eps, double* o, double* rstd);
int m2rnn_ref_gate_rmsnorm_backward(int ntok, int d, const double* y, const double* g, const double* w,
                                    double eps, const double* dout, double* dy, double* dg, double* dw);

/* Causal depthwise Conv1D of width 4 and SiLU before the scan (slide "Most of
 * the block can be computed before recurrence", paper Fig. 2): for u, z
 * [B][T][C], w [C][4], bias [C] (NULL: none),
 *   z[b][t][c] = silu(bias[c] + sum_{j=0..3} w[c][j] u[b][t-3+j][c]),
 * zero input before t = 0.  Backward from dz: du [B][T][C], dw [C][4] and
 * dbias [C] (NULL: not wanted) summed over b and t.  Return 0, -1 on a bad
 * argument, -2 when out of memory. */
int m2rnn_ref_conv_silu_forward(int B, int T, int C, const double* u, const double* w, const double* bias,
                                double* z);
int m2rnn_ref_conv_silu_backward(int B, int T, int C, const double* u, const double* w, const double* bias,
                                 const double* dz, double* du, double* dw, double* dbias);

#ifdef __cplusplus
}
#endif
#endif

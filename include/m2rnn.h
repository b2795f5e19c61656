/*
 * m2rnn.h -- C ABI of libm2rnn.so, the MI355X (gfx950) M2RNN scan.
 *
 * The operation, from the M2RNN paper-discussion slides (reading of
 * Mishra, Tan, Stoica, Gonzalez, Dao, arXiv:2603.14360v2):
 *
 *   slide "Write, transform, retain, and read a matrix state" (paper
 *   Eqs. (10)-(12)): for every batch row b and value head n, from H_0 = 0
 *   (the slides' start) or from a caller-given H_0 (the same recurrence
 *   resumed from a stored state, so a sequence can span several calls),
 *       Z_t = tanh(H_{t-1} W + k_t v_t^T)
 *       H_t = f_t H_{t-1} + (1 - f_t) Z_t
 *       y_t = H_t^T q_t + w_r (.) v_t
 *   H_t, Z_t are K x V (K = 64, V = 16), W is V x V, f_t a scalar per head.
 *
 *   slide "Shared queries and keys buy more recurrent capacity" (paper
 *   Alg. 1 / App. A): one q_t and one k_t per token, shared by the N value
 *   heads; v, f, W and w_r are per head.
 *
 *   slide "Backup: the recurrent gradient needs both paths": the backward
 *   (R_t = C_t + q_t u_t^T, D_t = ((1-f_t) R_t) (.) (1 - Z_t (.) Z_t),
 *   C_{t-1} = f_t R_t + D_t W^T, dL/df_t = <R_t, H_{t-1} - Z_t>,
 *   dL/dW = sum_t H_{t-1}^T D_t), completed by the plain chain rule for
 *   q, k, v and w_r.
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major (C-contiguous) DEVICE buffers owned by
 *     the caller.  The library never allocates, frees or synchronises.
 *     Between calls it keeps only the thread-local error message, the
 *     per-device address of its scratch array (m2rnn_gate_rmsnorm_backward_noalloc)
 *     and a per-device kernel attribute set on a device's first backward.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *     asynchronous on that stream; results are ready when it is.
 *   - Inputs q, k, v, f, W, w_r all have dtype `dtype` (M2RNN_F32 or
 *     M2RNN_BF16, bfloat16 as raw 16-bit words).  The state, every
 *     accumulation, y, H_T, checkpoints and all gradients are float32.
 *   - q, k, v, y, H_0, H_T, H_ckpt, dy, dH_T and every gradient buffer must
 *     be 16-byte aligned; f, W, w_r need their element alignment.
 *   - Outputs are fully overwritten; they need no zeroing.
 *   - Sizes: B, T, N >= 0.  B == 0 or N == 0 is a no-op.  T == 0 leaves
 *     y empty and sets H_T = H_0 (zero when H_0 is NULL) and dH_0 = dH_T
 *     (zero when dH_T is NULL).  This build supports K == 64 and
 *     V == 16 only (other values return M2RNN_ERR_UNSUPPORTED).
 *   - Size limits (beyond them M2RNN_ERR_UNSUPPORTED; each keeps a kernel
 *     launch under 2^32 work-items): B T N V <= 2^40; B ceil(N/4) < 2^22,
 *     about 16.7 M (b, n) chains or 64 GiB of state; and in the backward,
 *     when ckpt_every > 4, B ceil(N/4) ceil(T/ckpt_every) < 2^24.  The
 *     workspace query returns 0 beyond the first two.
 *   - f is used as given (not clamped); the method expects f in [0, 1].
 *   - Precision with bf16 inputs: the forward keeps the fp32 state to an
 *     fp16 hi/lo pair (2^-22 relative) in its H W contraction, and the
 *     backward's reverse sweep rounds its factors once to fp16 (see
 *     m2rnn_backward), so W must lie within fp16's range, |W| <= 65504
 *     (entries below 2^-14 in magnitude round to within 2^-25; entries
 *     beyond the range make the results non-finite).  fp32 inputs use exact
 *     fp32 products throughout.  tanh is 1 - 2 / (1 + 2^{2x / ln 2}) with the
 *     hardware exp2 and reciprocal: within 2.5e-7 of tanh (measured over
 *     [-10, 10], |x| < 1e-3 and |x| >= 20), exactly +-1 for |x| >= 20.
 *   - Errors are reported before anything is launched: a negative status is
 *     returned and m2rnn_last_error() describes it.  A failed kernel launch
 *     returns M2RNN_ERR_HIP.
 */
#ifndef M2RNN_H
#define M2RNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  M2RNN_OK = 0,
  M2RNN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative size, bad dtype */
  M2RNN_ERR_UNSUPPORTED = -2, /* K != 64 or V != 16, or a size beyond the limits */
  M2RNN_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  M2RNN_ERR_HIP = -4          /* the HIP runtime reported an error */
} m2rnn_status;

typedef enum { M2RNN_F32 = 0, M2RNN_BF16 = 1 } m2rnn_dtype;

/*
 * Forward scan (slide "Write, transform, retain, and read a matrix state",
 * paper Eqs. (10)-(12)).
 *   q, k    [B][T][K]     inputs, shared by the N heads of batch row b
 *   v       [B][T][N][V]
 *   f       [B][T][N]
 *   W       [N][V][V]     (H W)[i][j] = sum_l H[i][l] * W[n][l][j]
 *   w_r     [N][V]
 *   H_0     [B][N][K][V]  float32 initial state, or NULL for zero
 *   y       [B][T][N][V]  float32 out, readout of the updated state H_t
 *   H_T     [B][N][K][V]  float32 out, state after step T
 *   H_ckpt  [B][N][ceil(T/ckpt_every)][K][V] float32 out, H at
 *           t = j * ckpt_every (j = 0 gives H_0); NULL with
 *           ckpt_every == 0 stores none.  These are what m2rnn_backward
 *           restarts its recompute from.
 *   workspace  m2rnn_forward_workspace_bytes(B, T, N, K, V) bytes of device
 *           memory, 256-byte aligned, contents on entry ignored; may be NULL
 *           when that is 0 (else M2RNN_ERR_WORKSPACE).
 * H_T may be the same buffer as H_0 (each state tile is read before it is
 * overwritten); no other outputs may overlap the inputs.
 *
 * Few chains (B N <= 128) take a forward that spreads each head's 64 rows over
 * 16 waves, one state element per lane, with exact fp32 products in H W (for
 * bf16 inputs too); a head's rows then span four workgroups, whose readout
 * partial sums go through the workspace (B N T 256 bytes) and are added in a
 * fixed order.  More chains need no workspace.  Either way the results are
 * bitwise the same from run to run.
 */
int m2rnn_forward(int B, int T, int N, int K, int V, int dtype,
                  const void* q, const void* k, const void* v, const void* f,
                  const void* W, const void* w_r, const float* H_0,
                  float* y, float* H_T, float* H_ckpt, int ckpt_every,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace m2rnn_forward and m2rnn_forward_gated need for
 * these sizes (0 if none, and for sizes they reject). */
size_t m2rnn_forward_workspace_bytes(int B, int T, int N, int K, int V);

/*
 * Forward scan with the forget gate computed in the kernel from a
 * pre-activation (slide "The gate preserves a direct path through time",
 * paper Eqs. (13), (17)):
 *       f_t = exp(-alpha[n] * softplus(a_t + beta[n]))
 * which for alpha = 1 is sigmoid(-(a_t + beta)); f lies in [0, 1] for
 * alpha >= 0 and is 1 everywhere for alpha = 0.
 *   a       [B][T][N]     gate pre-activation (dtype `dtype`), in place of f
 *   alpha   [N], beta [N] per-head gate parameters (dtype `dtype`)
 * Every other argument, and the result for the same f, as m2rnn_forward.
 */
int m2rnn_forward_gated(int B, int T, int N, int K, int V, int dtype,
                        const void* q, const void* k, const void* v, const void* a,
                        const void* alpha, const void* beta,
                        const void* W, const void* w_r, const float* H_0,
                        float* y, float* H_T, float* H_ckpt, int ckpt_every,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace m2rnn_backward and m2rnn_backward_gated need
 * for these sizes (0 if none).
 */
size_t m2rnn_backward_workspace_bytes(int B, int T, int N, int K, int V, int ckpt_every);

/*
 * Backward scan: gradients of L = sum(y * dy) + sum(H_T * dH_T) (slide
 * "Backup: the recurrent gradient needs both paths", plus the chain rule
 * for q, k, v, w_r).
 *   q, k, v, f, W, w_r   the forward's inputs (dtype `dtype`)
 *   H_ckpt, ckpt_every   the forward's checkpoints (ckpt_every >= 1); the
 *                        first holds the forward's H_0
 *   dy      [B][T][N][V] float32
 *   dH_T    [B][N][K][V] float32, or NULL for zero
 *   dq, dk  [B][T][K]    float32 out, summed over the N heads
 *   dv      [B][T][N][V] float32 out
 *   df      [B][T][N]    float32 out
 *   dW      [N][V][V]    float32 out, summed over batch rows and time
 *   dw_r    [N][V]       float32 out, summed over batch rows and time
 *   dH_0    [B][N][K][V] float32 out, dL/dH_0 (the end of the recursion for
 *                        C), or NULL when not wanted
 *   workspace            device buffer of at least
 *                        m2rnn_backward_workspace_bytes(...) bytes,
 *                        256-byte aligned; contents on entry are ignored
 * With bf16 inputs the reverse sweep rounds its factors once to fp16 (and,
 * when ckpt_every > 4, restarts every 4 steps from states the replay of the
 * checkpoint chunks computed at full precision and stored in fp16) and
 * first scales dy and dH_T by the power of two that puts their largest
 * magnitude in [1/4, 1/2), scaling every output back exactly: the results
 * do not depend on the scale of the caller's gradients (dy, dH_T times 2^k
 * give every output times 2^k, bit for bit).  NaNs in dy are left out of
 * that scale and reach the outputs as usual.
 */
int m2rnn_backward(int B, int T, int N, int K, int V, int dtype,
                   const void* q, const void* k, const void* v, const void* f,
                   const void* W, const void* w_r,
                   const float* H_ckpt, int ckpt_every,
                   const float* dy, const float* dH_T,
                   float* dq, float* dk, float* dv, float* df,
                   float* dW, float* dw_r, float* dH_0,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward scan of m2rnn_forward_gated: the gradients of m2rnn_backward with
 * df carried through the gate (slide "The gate preserves a direct path
 * through time", paper Eqs. (13), (17)): with s = softplus(a_t + beta[n]),
 *       da_t     = df_t * f_t * (-alpha[n]) * sigmoid(a_t + beta[n])
 *       dalpha[n] = sum over b, t of df_t * f_t * (-s)
 *       dbeta[n]  = sum over b, t of da_t
 *   a, alpha, beta       the forward's gate inputs (dtype `dtype`)
 *   da      [B][T][N]    float32 out, in place of df
 *   dalpha, dbeta [N]    float32 out, 4-byte aligned
 * Every other argument as m2rnn_backward; the same workspace size.
 */
int m2rnn_backward_gated(int B, int T, int N, int K, int V, int dtype,
                         const void* q, const void* k, const void* v, const void* a,
                         const void* alpha, const void* beta,
                         const void* W, const void* w_r,
                         const float* H_ckpt, int ckpt_every,
                         const float* dy, const float* dH_T,
                         float* dq, float* dk, float* dv, float* da,
                         float* dalpha, float* dbeta, float* dW, float* dw_r, float* dH_0,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal Conv1D of width 4 and SiLU that q, k and v pass before the scan
 * (slide "Most of the block can be computed before recurrence", paper Fig. 2),
 * read as a depthwise convolution over time per channel with zero input
 * before t = 0 and taps in cross-correlation order (torch conv1d's):
 *       z[b][t][c] = silu(bias[c] + sum_{j=0..3} w[c][j] u[b][t-3+j][c])
 *   u     [B][T][C]  input (dtype `dtype`), e.g. a projected q, k or v with
 *                    C = 64, 64 or N V; 4-element aligned
 *   w     [C][4]     taps (dtype `dtype`), 4-element aligned
 *   bias  [C]        (dtype `dtype`) or NULL for none
 *   z     [B][T][C]  out, dtype `dtype` (bf16: rounded to nearest even from
 *                    the float32 result); must not overlap u
 * C must be a multiple of 4 (else M2RNN_ERR_UNSUPPORTED).
 */
int m2rnn_conv_silu_forward(int B, int T, int C, int dtype, const void* u, const void* w,
                            const void* bias, void* z, void* stream);

/* Bytes of device workspace m2rnn_conv_silu_backward needs (0 if none). */
size_t m2rnn_conv_silu_backward_workspace_bytes(int B, int T, int C);

/*
 * Backward of m2rnn_conv_silu_forward by the chain rule: with
 * a = bias + sum_j w[c][j] u[t-3+j] and silu'(a) = s (1 + a (1 - s)),
 * s = 1 / (1 + e^{-a}), da = dz silu'(a) and
 *       du[b][t][c] = sum_j w[c][j] da[b][t+3-j][c]      (zero past T)
 *       dw[c][j] = sum_{b,t} da[b][t][c] u[b][t-3+j][c],  dbias[c] = sum_{b,t} da
 *   u, w, bias     the forward's inputs
 *   dz    [B][T][C] float32, 16-byte aligned
 *   du    [B][T][C] float32 out; must not overlap dz
 *   dw    [C][4] float32 out; dbias [C] float32 out or NULL (not wanted);
 *                  both summed over b and t in a fixed order
 *   workspace      m2rnn_conv_silu_backward_workspace_bytes(...) bytes,
 *                  16-byte aligned; contents on entry are ignored
 * B T == 0 sets dw (and dbias) to 0.
 */
int m2rnn_conv_silu_backward(int B, int T, int C, int dtype, const void* u, const void* w,
                             const void* bias, const float* dz, float* du, float* dw, float* dbias,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Output gate and RMSNorm after the readout (slide "Most of the block can be
 * computed before recurrence", paper Fig. 2), with the per-token statistic of
 * slide "Backup: RMSNormTP synchronizes per-token statistics" (paper App. C,
 * Eqs. (26)-(33)) over the token's d = N V features on this GPU:
 *       x = y (.) g,   s = ((1/d) sum_j x_j^2 + eps)^{-1/2},   out = w (.) x s
 * (the pages omit eps: eps = 0 is their form; a token whose x is all zero
 * then gives non-finite output).
 *   y     [B][T][N][V] float32 (the scan's readout)
 *   g     [B][T][N][V] output gate (dtype `dtype`), 4-element aligned
 *   w     [N][V]       RMSNorm weight (dtype `dtype`), 4-element aligned
 *   eps   >= 0, finite
 *   out   [B][T][N][V] float32 out; may be the same buffer as y
 *   rstd  [B][T] float32 out (s of each token), or NULL
 * N V must be a multiple of 4 and at most 2048 (else M2RNN_ERR_UNSUPPORTED).
 */
int m2rnn_gate_rmsnorm_forward(int B, int T, int N, int V, int dtype,
                               const float* y, const void* g, const void* w, float eps,
                               float* out, float* rstd, void* stream);

/* Bytes of device workspace m2rnn_gate_rmsnorm_backward needs (0 if none). */
size_t m2rnn_gate_rmsnorm_backward_workspace_bytes(int B, int T, int N, int V);

/*
 * Backward of m2rnn_gate_rmsnorm_forward, as on slide "Backup: RMSNormTP
 * synchronizes per-token statistics": with p = w (.) dout and
 * r = sum_j p_j x_j per token, dx = s p - (r s^3 / d) x, and then
 *       dy = dx (.) g,   dg = dx (.) y,   dw = sum over tokens of dout (.) x s.
 *   y, g, w, eps   the forward's inputs
 *   dout  [B][T][N][V] float32
 *   dy, dg [B][T][N][V] float32 out (dy may be the same buffer as dout)
 *   dw    [N][V] float32 out, summed over tokens in a fixed order
 *   workspace      m2rnn_gate_rmsnorm_backward_workspace_bytes(...) bytes,
 *                  16-byte aligned; contents on entry are ignored
 * B T == 0 sets dw = 0.
 */
int m2rnn_gate_rmsnorm_backward(int B, int T, int N, int V, int dtype,
                                const float* y, const void* g, const void* w, float eps,
                                const float* dout, float* dy, float* dg, float* dw,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * m2rnn_gate_rmsnorm_backward for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, and the same
 * results and errors.  Its dw partial sums go to a scratch array inside the
 * library, 8,650,752 bytes on each GPU it runs on (held until the process
 * ends), which covers every size the entry point accepts (N V <= 2048);
 * a workspace beyond it would return M2RNN_ERR_UNSUPPORTED.  The GPU is the
 * one `stream` belongs to (the current device for the NULL stream).  It calls
 * no allocation routine.  All calls on one GPU share that GPU's array: calls
 * that may run at the same time on one GPU (different streams, or different
 * host threads without ordering) race on it and give wrong dw; order them on
 * one stream.
 */
int m2rnn_gate_rmsnorm_backward_noalloc(int B, int T, int N, int V, int dtype,
                                        const float* y, const void* g, const void* w, float eps,
                                        const float* dout, float* dy, float* dg, float* dw,
                                        void* stream);

/*
 * One token of the recurrence for every (b, n), state held by the caller
 * (decoding): the forward of slide "Write, transform, retain, and read a
 * matrix state" for T = 1 from H, with H overwritten by the new state.
 *   q, k  [B][K]; v [B][N][V]; f [B][N]; W [N][V][V]; w_r [N][V] (dtype)
 *   H     [B][N][K][V] float32 in/out
 *   y     [B][N][V]    float32 out
 * Same as m2rnn_forward with T = 1, H_0 = H_T = H and no checkpoints, and
 * bit-identical to the first step of that forward at four heads of one wave
 * each (more than 1536 chains); one wave per head reads its state, steps and
 * writes it back, with no staging and no workspace.  q, k, v, H and y must be
 * 16-byte aligned, f, W and w_r element-aligned.
 */
int m2rnn_decode(int B, int N, int K, int V, int dtype,
                 const void* q, const void* k, const void* v, const void* f,
                 const void* W, const void* w_r, float* H, float* y, void* stream);

/* Message for the last non-OK status on the calling thread ("" if none). */
const char* m2rnn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* M2RNN_H */

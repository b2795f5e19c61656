// m2rnn_api.hip -- the C ABI of libm2rnn.so (declared in include/m2rnn.h):
// argument validation, error reporting and kernel dispatch.  No allocation,
// no synchronisation, no state beyond the thread-local error message.
#include "m2rnn.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "m2rnn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Largest element count any single tensor may have (64-bit indexing is used in
// the kernels; this only keeps products of int sizes from overflowing).
constexpr long long kMaxElems = 1LL << 40;
// A launch holds fewer than 2^32 work-items.  The backward's workgroups of four
// heads have 1024 threads, the replay's 256 per checkpoint interval: these
// bound the groups of four heads, and the backward's groups times intervals.
constexpr long long kMaxHeadGroups = (1LL << 22) - 1;
constexpr long long kMaxReplayGroups = (1LL << 24) - 1;

// True when the product of non-negative sizes exceeds `limit`; the product is
// formed in 128 bits, where four int factors cannot overflow.
bool too_large(long long limit, long long a, long long b, long long c = 1, long long d = 1) {
  return (__int128)a * b * c * d > limit;
}

int check_sizes(int B, int T, int N, int K, int V, int dtype) {
  if (B < 0 || T < 0 || N < 0) return fail(M2RNN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d T=%d N=%d)", B, T, N);
  if (K != 64 || V != 16) return fail(M2RNN_ERR_UNSUPPORTED, "this build supports K=64, V=16 only (got K=%d V=%d)", K, V);
  if (dtype != M2RNN_F32 && dtype != M2RNN_BF16) return fail(M2RNN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (too_large(kMaxElems, B, T, N, V)) return fail(M2RNN_ERR_UNSUPPORTED, "problem too large");
  if ((long long)B * (((long long)N + 3) / 4) > kMaxHeadGroups)
    return fail(M2RNN_ERR_UNSUPPORTED, "B * ceil(N / 4) must be below 2^22 (B=%d N=%d)", B, N);
  return M2RNN_OK;
}

// Check a required device pointer: non-null when the tensor is non-empty, and
// aligned to `align` bytes.
int need(const void* p, const char* name, long long elems, size_t align) {
  if (elems <= 0) return M2RNN_OK;
  if (!p) return fail(M2RNN_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned(p, align)) return fail(M2RNN_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return M2RNN_OK;
}

}  // namespace

extern "C" const char* m2rnn_last_error(void) { return g_err; }

extern "C" size_t m2rnn_forward_workspace_bytes(int B, int T, int N, int K, int V) {
  if (B <= 0 || T <= 0 || N <= 0 || K != 64 || V != 16) return 0;
  if (too_large(kMaxElems, B, T, N, V) || (long long)B * (((long long)N + 3) / 4) > kMaxHeadGroups) return 0;
  return sizeof(float) * m2rnn::forward_workspace_floats(B, T, N);
}

// f is given, or computed from the gate pre-activation ga and (galpha, gbeta).
// `workspace` feeds the row-split forward (few chains).
static int forward_impl(bool gated, int B, int T, int N, int K, int V, int dtype, const void* q, const void* k,
                        const void* v, const void* f, const void* ga, const void* galpha, const void* gbeta,
                        const void* W, const void* w_r, const float* H_0, float* y, float* H_T, float* H_ckpt,
                        int ckpt_every, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int st = check_sizes(B, T, N, K, V, dtype);
  if (st) return st;
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  const long long BT = (long long)B * T, BTN = BT * N, BN = (long long)B * N;
  if (ckpt_every < 0) return fail(M2RNN_ERR_INVALID_ARG, "ckpt_every must be >= 0");
  if ((H_ckpt != nullptr) != (ckpt_every > 0))
    return fail(M2RNN_ERR_INVALID_ARG, "H_ckpt and ckpt_every > 0 go together");
  if ((st = need(q, "q", BT * K, 16)) || (st = need(k, "k", BT * K, 16)) || (st = need(v, "v", BTN * V, 16)) ||
      (st = need(gated ? ga : f, gated ? "a" : "f", BTN, es)) ||
      (st = need(galpha, "alpha", gated ? (long long)N * (BN > 0) : 0, es)) ||
      (st = need(gbeta, "beta", gated ? (long long)N * (BN > 0) : 0, es)) ||
      (st = need(W, "W", (long long)N * V * V * (BN > 0), es)) ||
      (st = need(w_r, "w_r", (long long)N * V * (BN > 0), es)) || (st = need(y, "y", BTN * V, 16)) ||
      (st = need(H_T, "H_T", BN * K * V, 16)))
    return st;
  if (H_0 && !aligned(H_0, 16)) return fail(M2RNN_ERR_INVALID_ARG, "H_0 must be 16-byte aligned");
  const int nck = ckpt_every > 0 ? (int)(((long long)T + ckpt_every - 1) / ckpt_every) : 0;
  if (ckpt_every > 0 && (st = need(H_ckpt, "H_ckpt", BN * nck * K * V, 16))) return st;
  if (BN == 0) return M2RNN_OK;

  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {  // H_T = H_0; y is empty
    hipError_t e = H_0 ? m2rnn::launch_copy(H_T, H_0, (size_t)BN * K * V, s)
                       : m2rnn::launch_fill_zero(H_T, (size_t)BN * K * V, s);
    return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "H_T = H_0: %s", hipGetErrorString(e));
  }
  m2rnn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.f = f; a.W = W; a.wr = w_r; a.H_0 = H_0;
  if (gated) { a.ga = ga; a.galpha = galpha; a.gbeta = gbeta; }
  a.y = y; a.H_T = H_T; a.H_ckpt = ckpt_every > 0 ? H_ckpt : nullptr;
  a.B = B; a.T = T; a.N = N; a.ckpt_every = ckpt_every; a.nck = nck;
  const size_t ws_need = sizeof(float) * m2rnn::forward_workspace_floats(B, T, N);
  hipError_t e;
  if (ws_need > 0) {
    if (!workspace || workspace_bytes < ws_need)
      return fail(M2RNN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws_need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(M2RNN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    a.ypart = (float*)workspace;
    e = m2rnn::launch_forward_rows(a, dtype, s);
  } else {
    e = m2rnn::launch_forward(a, dtype, s);
  }
  if (e != hipSuccess) return fail(M2RNN_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return M2RNN_OK;
}

extern "C" int m2rnn_forward(int B, int T, int N, int K, int V, int dtype, const void* q, const void* k,
                             const void* v, const void* f, const void* W, const void* w_r, const float* H_0,
                             float* y, float* H_T, float* H_ckpt, int ckpt_every, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return forward_impl(false, B, T, N, K, V, dtype, q, k, v, f, nullptr, nullptr, nullptr, W, w_r, H_0, y, H_T, H_ckpt,
                      ckpt_every, workspace, workspace_bytes, stream);
}

extern "C" int m2rnn_forward_gated(int B, int T, int N, int K, int V, int dtype, const void* q, const void* k,
                                   const void* v, const void* a, const void* alpha, const void* beta,
                                   const void* W, const void* w_r, const float* H_0, float* y, float* H_T,
                                   float* H_ckpt, int ckpt_every, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return forward_impl(true, B, T, N, K, V, dtype, q, k, v, nullptr, a, alpha, beta, W, w_r, H_0, y, H_T, H_ckpt,
                      ckpt_every, workspace, workspace_bytes, stream);
}

extern "C" size_t m2rnn_backward_workspace_bytes(int B, int T, int N, int K, int V, int ckpt_every) {
  if (B <= 0 || T <= 0 || N <= 0 || K != 64 || V != 16 || ckpt_every < 1) return 0;
  if (too_large(kMaxElems, B, T, N, V) || (long long)B * (((long long)N + 3) / 4) > kMaxHeadGroups) return 0;
  size_t o1, o2, o3, o4, o5, o6;
  int ng;
  return sizeof(float) * m2rnn::backward_workspace_floats(B, T, N, ckpt_every, &o1, &o2, &o3, &o4, &o5, &o6, &ng);
}

// f is given (df out) or computed from the gate (da in the df slot, dalpha and
// dbeta out).
static int backward_impl(bool gated, int B, int T, int N, int K, int V, int dtype, const void* q, const void* k, const void* v,
                         const void* f, const void* ga, const void* galpha, const void* gbeta, const void* W,
                         const void* w_r, const float* H_ckpt, int ckpt_every, const float* dy, const float* dH_T,
                         float* dq, float* dk, float* dv, float* df, float* dalpha, float* dbeta, float* dW,
                         float* dw_r, float* dH_0, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int st = check_sizes(B, T, N, K, V, dtype);
  if (st) return st;
  if (ckpt_every < 1) return fail(M2RNN_ERR_INVALID_ARG, "ckpt_every must be >= 1 for the backward");
  if (ckpt_every > m2rnn::backward_sub_steps() &&
      (long long)B * (((long long)N + 3) / 4) * ((T + (long long)ckpt_every - 1) / ckpt_every) > kMaxReplayGroups)
    return fail(M2RNN_ERR_UNSUPPORTED, "B * ceil(N / 4) * ceil(T / ckpt_every) must be below 2^24");
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  const long long BT = (long long)B * T, BTN = BT * N, BN = (long long)B * N;
  const int nck = T > 0 ? (int)(((long long)T + ckpt_every - 1) / ckpt_every) : 0;
  if ((st = need(q, "q", BT * K * (N > 0), 16)) || (st = need(k, "k", BT * K * (N > 0), 16)) ||
      (st = need(v, "v", BTN * V, 16)) || (st = need(gated ? ga : f, gated ? "a" : "f", BTN, es)) ||
      (st = need(galpha, "alpha", gated ? (long long)N : 0, es)) ||
      (st = need(gbeta, "beta", gated ? (long long)N : 0, es)) ||
      (st = need(dalpha, "dalpha", gated ? (long long)N : 0, 4)) ||
      (st = need(dbeta, "dbeta", gated ? (long long)N : 0, 4)) ||
      (st = need(W, "W", (long long)N * V * V, es)) ||
      (st = need(w_r, "w_r", (long long)N * V, es)) || (st = need(H_ckpt, "H_ckpt", BN * nck * K * V, 16)) ||
      (st = need(dy, "dy", BTN * V, 16)) || (st = need(dq, "dq", BT * K, 16)) || (st = need(dk, "dk", BT * K, 16)) ||
      (st = need(dv, "dv", BTN * V, 16)) || (st = need(df, gated ? "da" : "df", BTN, 4)) || (st = need(dW, "dW", (long long)N * V * V, 16)) ||
      (st = need(dw_r, "dw_r", (long long)N * V, 16)))
    return st;
  if (dH_T && !aligned(dH_T, 16)) return fail(M2RNN_ERR_INVALID_ARG, "dH_T must be 16-byte aligned");
  if (dH_0 && !aligned(dH_0, 16)) return fail(M2RNN_ERR_INVALID_ARG, "dH_0 must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (BTN == 0) {
    // nothing flows back through the steps: dq, dk (if any) and the summed
    // dW, dw_r are zero, and dH_0 = dH_T
    hipError_t e = hipSuccess;
    if (dH_0 && BN > 0)
      e = dH_T ? m2rnn::launch_copy(dH_0, dH_T, (size_t)BN * K * V, s) : m2rnn::launch_fill_zero(dH_0, (size_t)BN * K * V, s);
    if (BT > 0) {
      if (e == hipSuccess) e = m2rnn::launch_fill_zero(dq, (size_t)BT * K, s);
      if (e == hipSuccess) e = m2rnn::launch_fill_zero(dk, (size_t)BT * K, s);
    }
    if (N > 0) {
      if (e == hipSuccess) e = m2rnn::launch_fill_zero(dW, (size_t)N * V * V, s);
      if (e == hipSuccess) e = m2rnn::launch_fill_zero(dw_r, (size_t)N * V, s);
      if (gated && e == hipSuccess) e = m2rnn::launch_fill_zero(dalpha, (size_t)N, s);
      if (gated && e == hipSuccess) e = m2rnn::launch_fill_zero(dbeta, (size_t)N, s);
    }
    return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "zero fill: %s", hipGetErrorString(e));
  }
  size_t o_dense, o_dqk, o_dW, o_dwr, o_dgate, o_amax;
  int ng;
  const size_t need_bytes = sizeof(float) * m2rnn::backward_workspace_floats(B, T, N, ckpt_every, &o_dense, &o_dqk,
                                                                              &o_dW, &o_dwr, &o_dgate, &o_amax, &ng);
  if (!workspace || workspace_bytes < need_bytes)
    return fail(M2RNN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(M2RNN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  float* ws = (float*)workspace;
  m2rnn::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.f = f; a.W = W; a.wr = w_r;
  a.H_ckpt = H_ckpt; a.dy = dy; a.dH_T = dH_T;
  a.dq = dq; a.dk = dk; a.dv = dv; a.df = df; a.dW = dW; a.dw_r = dw_r; a.dH_0 = dH_0;
  a.ws_dqk = ws + o_dqk; a.ws_dW = ws + o_dW; a.ws_dwr = ws + o_dwr; a.ws_dgate = ws + o_dgate;
  a.ws_amax = ws + o_amax;
  if (gated) { a.ga = ga; a.galpha = galpha; a.gbeta = gbeta; a.dalpha = dalpha; a.dbeta = dbeta; }
  a.B = B; a.T = T; a.N = N;
  a.ckpt_every = ckpt_every; a.nck = nck; a.ngroups = ng;
  // replay of the caller's checkpoint chunks into states every sub-step count
  const int L = m2rnn::backward_sub_steps();
  m2rnn::FwdArgs rp;
  rp.q = q; rp.k = k; rp.v = v; rp.f = f; rp.W = W; rp.wr = w_r;
  if (gated) { rp.ga = ga; rp.galpha = galpha; rp.gbeta = gbeta; }
  rp.y = nullptr; rp.H_T = nullptr; rp.H_ckpt = ws + o_dense;
  rp.B = B; rp.T = T; rp.N = N; rp.ckpt_every = L; rp.nck = (int)(((long long)T + L - 1) / L);
  rp.H_src = H_ckpt; rp.src_every = ckpt_every; rp.src_nck = nck;
  hipError_t e = m2rnn::launch_backward(a, rp, dtype, s);
  if (e != hipSuccess) return fail(M2RNN_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return M2RNN_OK;
}

extern "C" int m2rnn_backward(int B, int T, int N, int K, int V, int dtype, const void* q, const void* k,
                              const void* v, const void* f, const void* W, const void* w_r, const float* H_ckpt,
                              int ckpt_every, const float* dy, const float* dH_T, float* dq, float* dk, float* dv,
                              float* df, float* dW, float* dw_r, float* dH_0, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return backward_impl(false, B, T, N, K, V, dtype, q, k, v, f, nullptr, nullptr, nullptr, W, w_r, H_ckpt, ckpt_every, dy,
                       dH_T, dq, dk, dv, df, nullptr, nullptr, dW, dw_r, dH_0, workspace, workspace_bytes, stream);
}

extern "C" int m2rnn_backward_gated(int B, int T, int N, int K, int V, int dtype, const void* q, const void* k,
                                    const void* v, const void* a, const void* alpha, const void* beta,
                                    const void* W, const void* w_r, const float* H_ckpt, int ckpt_every,
                                    const float* dy, const float* dH_T, float* dq, float* dk, float* dv, float* da,
                                    float* dalpha, float* dbeta, float* dW, float* dw_r, float* dH_0,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(true, B, T, N, K, V, dtype, q, k, v, nullptr, a, alpha, beta, W, w_r, H_ckpt, ckpt_every, dy,
                       dH_T, dq, dk, dv, da, dalpha, dbeta, dW, dw_r, dH_0, workspace, workspace_bytes, stream);
}

extern "C" int m2rnn_decode(int B, int N, int K, int V, int dtype, const void* q, const void* k, const void* v,
                            const void* f, const void* W, const void* w_r, float* H, float* y, void* stream) {
  g_err[0] = 0;
  int st = check_sizes(B, 1, N, K, V, dtype);
  if (st) return st;
  const long long BN = (long long)B * N;
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  if ((st = need(H, "H", BN * K * V, 16)) || (st = need(q, "q", BN > 0 ? (long long)B * K : 0, 16)) ||
      (st = need(k, "k", BN > 0 ? (long long)B * K : 0, 16)) || (st = need(v, "v", BN * V, 16)) ||
      (st = need(f, "f", BN, es)) || (st = need(W, "W", BN > 0 ? (long long)N * V * V : 0, es)) ||
      (st = need(w_r, "w_r", BN > 0 ? (long long)N * V : 0, es)) || (st = need(y, "y", BN * V, 16)))
    return st;
  if (BN == 0) return M2RNN_OK;
  m2rnn::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.f = f; a.W = W; a.wr = w_r; a.H = H; a.y = y;
  a.B = B; a.N = N;
  const hipError_t e = m2rnn::launch_decode(a, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(M2RNN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return M2RNN_OK;
}

// ------------------------------------------------- output gate and RMSNorm
namespace {

int norm_check(int B, int T, int N, int V, int dtype, float eps, long long* ntok, int* d) {
  if (B < 0 || T < 0 || N < 0 || V < 0)
    return fail(M2RNN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d T=%d N=%d V=%d)", B, T, N, V);
  if (dtype != M2RNN_F32 && dtype != M2RNN_BF16) return fail(M2RNN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(M2RNN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const long long dd = (long long)N * V;
  if (dd % 4 != 0 || dd > m2rnn::kNormMaxD)
    return fail(M2RNN_ERR_UNSUPPORTED, "N*V must be a multiple of 4 and at most %d (got %lld)", m2rnn::kNormMaxD, dd);
  if (too_large(kMaxElems, B, T, dd)) return fail(M2RNN_ERR_UNSUPPORTED, "problem too large");
  *ntok = (long long)B * T;
  *d = (int)dd;
  return M2RNN_OK;
}

}  // namespace

extern "C" int m2rnn_gate_rmsnorm_forward(int B, int T, int N, int V, int dtype, const float* y, const void* g,
                                          const void* w, float eps, float* out, float* rstd, void* stream) {
  g_err[0] = 0;
  long long ntok;
  int d, st;
  if ((st = norm_check(B, T, N, V, dtype, eps, &ntok, &d))) return st;
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  const long long n = ntok * d;
  if ((st = need(y, "y", n, 16)) || (st = need(g, "g", n, 4 * es)) || (st = need(w, "w", n > 0 ? d : 0, 4 * es)) ||
      (st = need(out, "out", n, 16)))
    return st;
  if (rstd && !aligned(rstd, 4)) return fail(M2RNN_ERR_INVALID_ARG, "rstd must be 4-byte aligned");
  if (n == 0) return M2RNN_OK;
  m2rnn::NormArgs a{};
  a.y = y; a.g = g; a.w = w; a.out = out; a.rstd = rstd; a.ntok = ntok; a.d = d; a.eps = eps;
  hipError_t e = m2rnn::launch_norm_forward(a, dtype, (hipStream_t)stream);
  return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "gate_rmsnorm forward launch: %s", hipGetErrorString(e));
}

extern "C" size_t m2rnn_gate_rmsnorm_backward_workspace_bytes(int B, int T, int N, int V) {
  if (B < 0 || T < 0 || N < 0 || V < 0) return 0;
  const long long ntok = (long long)B * T, d = (long long)N * V;
  if (ntok == 0 || d == 0 || d % 4 != 0 || d > m2rnn::kNormMaxD) return 0;
  return sizeof(float) * m2rnn::norm_backward_workspace_floats(ntok, (int)d);
}

namespace {

// Validation shared by both backward entry points.  Returns M2RNN_OK with
// *done set when nothing needs a workspace (d == 0, or B T == 0 where dw = 0
// is written), else fills *a for the launch.
int norm_backward_prepare(int B, int T, int N, int V, int dtype, const float* y, const void* g, const void* w,
                          float eps, const float* dout, float* dy, float* dg, float* dw, void* stream,
                          m2rnn::NormArgs* a, bool* done) {
  long long ntok;
  int d, st;
  *done = true;
  if ((st = norm_check(B, T, N, V, dtype, eps, &ntok, &d))) return st;
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  const long long n = ntok * d;
  if ((st = need(y, "y", n, 16)) || (st = need(g, "g", n, 4 * es)) || (st = need(w, "w", n > 0 ? d : 0, 4 * es)) ||
      (st = need(dout, "dout", n, 16)) || (st = need(dy, "dy", n, 16)) || (st = need(dg, "dg", n, 16)) ||
      (st = need(dw, "dw", d, 16)))
    return st;
  if (d == 0) return M2RNN_OK;
  if (ntok == 0) {   // dw = 0
    hipError_t e = m2rnn::launch_fill_zero(dw, (size_t)d, (hipStream_t)stream);
    return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "dw = 0: %s", hipGetErrorString(e));
  }
  *a = m2rnn::NormArgs{};
  a->y = y; a->g = g; a->w = w; a->dout = dout; a->dy = dy; a->dg = dg; a->dw = dw;
  a->ntok = ntok; a->d = d; a->eps = eps;
  *done = false;
  return M2RNN_OK;
}

int norm_backward_launch(const m2rnn::NormArgs& a, int dtype, void* stream) {
  hipError_t e = m2rnn::launch_norm_backward(a, dtype, (hipStream_t)stream);
  return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "gate_rmsnorm backward launch: %s", hipGetErrorString(e));
}

}  // namespace

extern "C" int m2rnn_gate_rmsnorm_backward(int B, int T, int N, int V, int dtype, const float* y, const void* g,
                                           const void* w, float eps, const float* dout, float* dy, float* dg,
                                           float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  m2rnn::NormArgs a;
  bool done;
  int st = norm_backward_prepare(B, T, N, V, dtype, y, g, w, eps, dout, dy, dg, dw, stream, &a, &done);
  if (st || done) return st;
  const size_t need_bytes = m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, V);
  if (!workspace || workspace_bytes < need_bytes)
    return fail(M2RNN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(M2RNN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  a.ws = (float*)workspace;
  return norm_backward_launch(a, dtype, stream);
}

// ---------------------- output gate and RMSNorm backward without a workspace
//
// For callers that cannot allocate device memory: the dw partial sums go to
// `scratch`, a file-scope device array (one copy per GPU, held from the
// library's load until the process ends), sized for the largest workspace the
// backward takes: kNormMaxGroups partial rows and kColsumRowBlocks second-level
// rows of at most kNormMaxD floats.  Every element the kernels read from it is
// written earlier in the same call, so nothing needs clearing.  Host code
// never names `scratch` in a launch or a copy: its host-side name is not a
// device address.  The address comes from hipGetSymbolAddress, taken once per
// device with that device current.
namespace {
constexpr size_t kNormScratchFloats =
    ((size_t)m2rnn::kNormMaxGroups + m2rnn::kColsumRowBlocks) * (size_t)m2rnn::kNormMaxD;
}  // namespace

static __device__ __align__(256) float scratch[kNormScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the GPU that `stream` runs on (the
// current device for the NULL stream).
int scratch_address(void* stream, float** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(M2RNN_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(M2RNN_ERR_UNSUPPORTED, "device %d: only devices 0..%d are served", dev,
                                                 kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(M2RNN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(M2RNN_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !p)
      return fail(M2RNN_ERR_HIP, "address of the scratch array on device %d: %s", dev, hipGetErrorString(e));
    if (e2 != hipSuccess) return fail(M2RNN_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(e2));
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return M2RNN_OK;
}

}  // namespace

extern "C" int m2rnn_gate_rmsnorm_backward_noalloc(int B, int T, int N, int V, int dtype, const float* y,
                                                   const void* g, const void* w, float eps, const float* dout,
                                                   float* dy, float* dg, float* dw, void* stream) {
  g_err[0] = 0;
  m2rnn::NormArgs a;
  bool done;
  int st = norm_backward_prepare(B, T, N, V, dtype, y, g, w, eps, dout, dy, dg, dw, stream, &a, &done);
  if (st || done) return st;
  const size_t need_bytes = m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, V);
  if (need_bytes > sizeof(scratch))
    return fail(M2RNN_ERR_UNSUPPORTED, "needs %zu bytes of scratch; the library holds %zu", need_bytes,
                sizeof(scratch));
  float* ws = nullptr;
  if ((st = scratch_address(stream, &ws))) return st;
  a.ws = ws;
  return norm_backward_launch(a, dtype, stream);
}

// ------------------------------------------------ causal Conv1D and SiLU
namespace {

int conv_check(int B, int T, int C, int dtype) {
  if (B < 0 || T < 0 || C < 0) return fail(M2RNN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d T=%d C=%d)", B, T, C);
  if (dtype != M2RNN_F32 && dtype != M2RNN_BF16) return fail(M2RNN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (C % 4 != 0 || C > (1 << 20)) return fail(M2RNN_ERR_UNSUPPORTED, "C must be a multiple of 4, at most 2^20 (got %d)", C);
  if (too_large(kMaxElems, B, T, C)) return fail(M2RNN_ERR_UNSUPPORTED, "problem too large");
  return M2RNN_OK;
}

}  // namespace

extern "C" int m2rnn_conv_silu_forward(int B, int T, int C, int dtype, const void* u, const void* w,
                                       const void* bias, void* z, void* stream) {
  g_err[0] = 0;
  int st = conv_check(B, T, C, dtype);
  if (st) return st;
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  const long long n = (long long)B * T * C;
  if ((st = need(u, "u", n, 4 * es)) || (st = need(w, "w", n > 0 ? (long long)C * 4 : 0, 4 * es)) ||
      (st = need(z, "z", n, 4 * es)))
    return st;
  if (bias && !aligned(bias, 4 * es)) return fail(M2RNN_ERR_INVALID_ARG, "bias must be %zu-byte aligned", 4 * es);
  if (n == 0) return M2RNN_OK;
  m2rnn::ConvArgs a{};
  a.u = u; a.w = w; a.bias = bias; a.z = z; a.B = B; a.T = T; a.C = C;
  hipError_t e = m2rnn::launch_conv_forward(a, dtype, (hipStream_t)stream);
  return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "conv_silu forward launch: %s", hipGetErrorString(e));
}

extern "C" size_t m2rnn_conv_silu_backward_workspace_bytes(int B, int T, int C) {
  if (B <= 0 || T <= 0 || C <= 0 || C % 4 != 0 || C > (1 << 20)) return 0;
  return sizeof(float) * m2rnn::conv_backward_workspace_floats(B, T, C);
}

extern "C" int m2rnn_conv_silu_backward(int B, int T, int C, int dtype, const void* u, const void* w,
                                        const void* bias, const float* dz, float* du, float* dw, float* dbias,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int st = conv_check(B, T, C, dtype);
  if (st) return st;
  const size_t es = dtype == M2RNN_F32 ? 4 : 2;
  const long long n = (long long)B * T * C;
  if ((st = need(u, "u", n, 4 * es)) || (st = need(w, "w", n > 0 ? (long long)C * 4 : 0, 4 * es)) ||
      (st = need(dz, "dz", n, 16)) || (st = need(du, "du", n, 16)) || (st = need(dw, "dw", (long long)C * 4, 16)))
    return st;
  if (bias && !aligned(bias, 4 * es)) return fail(M2RNN_ERR_INVALID_ARG, "bias must be %zu-byte aligned", 4 * es);
  if (dbias && !aligned(dbias, 16)) return fail(M2RNN_ERR_INVALID_ARG, "dbias must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (C == 0) return M2RNN_OK;
  if (n == 0) {   // dw = dbias = 0
    hipError_t e = m2rnn::launch_fill_zero(dw, (size_t)C * 4, s);
    if (e == hipSuccess && dbias) e = m2rnn::launch_fill_zero(dbias, (size_t)C, s);
    return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "dw = 0: %s", hipGetErrorString(e));
  }
  const size_t need_bytes = m2rnn_conv_silu_backward_workspace_bytes(B, T, C);
  if (!workspace || workspace_bytes < need_bytes)
    return fail(M2RNN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(M2RNN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  m2rnn::ConvArgs a{};
  a.u = u; a.w = w; a.bias = bias; a.dz = dz; a.du = du; a.dw = dw; a.dbias = dbias; a.ws = (float*)workspace;
  a.B = B; a.T = T; a.C = C; a.R = m2rnn::conv_backward_workers(B, T, C);
  hipError_t e = m2rnn::launch_conv_backward(a, dtype, s);
  return e == hipSuccess ? M2RNN_OK : fail(M2RNN_ERR_HIP, "conv_silu backward launch: %s", hipGetErrorString(e));
}

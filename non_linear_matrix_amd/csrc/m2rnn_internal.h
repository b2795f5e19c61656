// m2rnn_internal.h -- launch arguments shared by the C-ABI layer and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace m2rnn {

struct FwdArgs {
  const void *q, *k, *v, *f, *W, *wr;
  // forget gate from a pre-activation: when ga is set, f = exp(-alpha
  // softplus(ga + beta)) with alpha = galpha[n], beta = gbeta[n] (f unused)
  const void *ga = nullptr, *galpha = nullptr, *gbeta = nullptr;
  const float* H_0 = nullptr;  // initial state, nullptr for zero
  float *y, *H_T, *H_ckpt;
  int B, T, N;
  int ckpt_every;  // > 0 when H_ckpt != nullptr
  int nck;         // ceil(T / ckpt_every)
  // replay from stored states (backward): checkpoints H_src every src_every steps
  const float* H_src = nullptr;
  int src_every = 0, src_nck = 0;
  // row-split forward: per-row-group readout partials [B][N][4][T][16]
  float* ypart = nullptr;
  // replay: amax_wgs extra workgroups (the first ones) that compute the
  // backward's gradient scale (grad_absmax_part) while the replay runs
  const float* amax_dy = nullptr;
  const float* amax_dH = nullptr;
  size_t amax_ndy4 = 0, amax_ndh4 = 0;
  float* amax_part = nullptr;
  int amax_wgs = 0;
};

hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t stream);

// One token for every (b, n) head from the caller's state H [B][N][64][16],
// updated in place (m2rnn_decode.hip).
struct DecodeArgs {
  const void *q, *k, *v, *f, *W, *wr;
  float *H, *y;
  int B, N;
};
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);
// Few chains (B N <= kRowsMaxChains): the row-split forward, one state element
// per lane (m2rnn_fwd_rows.hip), which needs forward_workspace_floats(B, T, N)
// floats of workspace in a.ypart for its readout partials (0 for more chains).
constexpr long long kRowsMaxChains = 128;
size_t forward_workspace_floats(int B, int T, int N);
hipError_t launch_forward_rows(const FwdArgs& a, int dtype, hipStream_t stream);
// Replay every checkpoint chunk of H_src in parallel, writing H every
// ckpt_every steps into H_ckpt (no y, no H_T).
hipError_t launch_densify(const FwdArgs& a, int dtype, hipStream_t stream);

struct BwdArgs {
  const void *q, *k, *v, *f, *W, *wr;
  const void *ga = nullptr, *galpha = nullptr, *gbeta = nullptr;   // gate (see FwdArgs)
  const float *H_ckpt, *dy, *dH_T;  // H_ckpt: states every ckpt_every (<= sub-step count) steps
  float *dq, *dk, *dv, *df, *dW, *dw_r;   // with the gate, df holds da
  float* dH_0;                      // nullptr when not wanted
  float *dalpha = nullptr, *dbeta = nullptr;   // gate parameters' gradients
  float *ws_dqk, *ws_dW, *ws_dwr;   // workspace regions
  float* ws_dgate = nullptr;        // [B][N][2] per-row dalpha, dbeta partials
  float* ws_amax = nullptr;         // partial maxima of |dy|, |dH_T| (bf16 inputs)
  float ck_scale = 2.8853900817779268f;   // H_ckpt holds H (c = 2 / ln 2) or, from the replay, c H (1)
  int B, T, N;
  int ckpt_every, nck, ngroups;
};

// Workspace layout (in floats) for the backward; returns the total.
size_t backward_workspace_floats(int B, int T, int N, int ckpt_every, size_t* off_dense, size_t* off_dqk,
                                 size_t* off_dW, size_t* off_dwr, size_t* off_dgate, size_t* off_amax,
                                 int* ngroups);
// Steps between the states the reverse sweep restarts from.
int backward_sub_steps();
// When a.ckpt_every exceeds the sub-step count, `replay` (a densify launch
// from the caller's checkpoints into the workspace) runs first.
hipError_t launch_backward(const BwdArgs& a, const FwdArgs& replay, int dtype, hipStream_t stream);

// Output gate and RMSNorm after the readout: per token row of d features,
// x = y * g, s = ((1/d) sum x^2 + eps)^{-1/2}, out = w * x * s.
struct NormArgs {
  const float* y;
  const void *g, *w;       // input dtype
  const float* dout;       // backward
  float *out, *rstd;       // forward (rstd may be nullptr)
  float *dy, *dg, *dw;     // backward
  float* ws;               // backward: dw partials [nwg][d], then [32][d]
  long long ntok;
  int d;
  float eps;
};
constexpr int kNormMaxD = 2048;
constexpr int kNormMaxGroups = 1024;   // workgroups (dw partial rows) of the backward, at most
// Workgroups (and dw partial rows) of the backward, and its workspace.
int norm_backward_groups(long long ntok, int d);
size_t norm_backward_workspace_floats(long long ntok, int d);
hipError_t launch_norm_forward(const NormArgs& a, int dtype, hipStream_t stream);
hipError_t launch_norm_backward(const NormArgs& a, int dtype, hipStream_t stream);

// Causal depthwise Conv1D (width 4) and SiLU over time, per channel:
// z[b][t][c] = silu(bias[c] + sum_j w[c][j] u[b][t-3+j][c]).
struct ConvArgs {
  const void *u, *w, *bias;   // input dtype; bias may be nullptr
  void* z;                    // forward output, input dtype
  const float* dz;            // backward
  float *du, *dw, *dbias;     // backward (dbias may be nullptr)
  float* ws;                  // backward: partials [R][C*5], then [kColsumRowBlocks][C*5]
  int B, T, C;
  int R;                      // backward: workers per channel group
};
constexpr int kConvTaps = 4;
constexpr int kConvStrip = 16;   // time steps per thread (forward)
constexpr int kConvStripBwd = 8; // time steps per thread (backward)
int conv_backward_workers(int B, int T, int C);
size_t conv_backward_workspace_floats(int B, int T, int C);
hipError_t launch_conv_forward(const ConvArgs& a, int dtype, hipStream_t stream);
hipError_t launch_conv_backward(const ConvArgs& a, int dtype, hipStream_t stream);

// out[col] = sum over rows of in[row][col] for cols columns (a multiple of 4),
// rows summed in a fixed order (two levels; ws2 holds kColsumRowBlocks rows
// of cols floats).  Columns below cols_a go to out_a[col], the rest to
// out_b[col - cols_a].
constexpr int kColsumRowBlocks = 32;
hipError_t launch_colsum(const float* in, int rows, int cols, float* ws2, float* out_a, int cols_a, float* out_b,
                         hipStream_t stream);

// Zero `n` floats with a plain fill kernel (graph-capture friendly).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);
// dst[i] = src[i] for `n` floats with a plain copy kernel; dst == src is allowed.
hipError_t launch_copy(float* dst, const float* src, size_t n, hipStream_t stream);

}  // namespace m2rnn

// m2rnn_conv.hip -- causal Conv1D (width 4) and SiLU before the scan.
//
// q, k and v reach the scan through a linear projection, a causal Conv1D of
// width 4 and a SiLU (slide "Most of the block can be computed before
// recurrence", paper Fig. 2).  Read as a depthwise convolution over time per
// channel, zero input before t = 0, taps in cross-correlation order:
//     a[b][t][c] = bias[c] + sum_{j=0..3} w[c][j] u[b][t-3+j][c],   z = silu(a)
//     da = dz silu'(a),   du[t] = sum_j w[c][j] da[t+3-j],
//     dw[c][j] = sum_{b,t} da[t] u[t-3+j],   dbias[c] = sum_{b,t} da[t].
// A time-parallel stencil, HBM-bound: each thread owns four channels of one
// batch row over a strip of kConvStrip steps and keeps the three previous
// input rows in registers, so every input row is read about once.  Threads
// are numbered with the channel group fastest, so a wave reads whole rows.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

namespace {

__device__ __forceinline__ f4 load4(const float* p) { return *(const f4*)p; }
__device__ __forceinline__ f4 load4(const bf16_t* p) { return Vec4<bf16_t>::to_f4(*(const uint2*)p); }
__device__ __forceinline__ void store4(float* p, f4 v) { *(f4*)p = v; }
__device__ __forceinline__ void store4(bf16_t* p, f4 v) {
  const uint32_t u01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{v[0], v[1]}), bf16x2));
  const uint32_t u23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{v[2], v[3]}), bf16x2));
  *(uint2*)p = uint2{u01, u23};
}

__device__ __forceinline__ f4 sigmoid4(f4 a) {
  f4 s;
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a[i] * kLog2e));
  return s;
}

// The four channels' taps (tap j as a vector over the channels) and bias.
template <typename TIn>
struct ConvTaps {
  f4 w[kConvTaps];
  f4 b;
  __device__ void load(const ConvArgs& a, int c0) {
    const TIn* wp = (const TIn*)a.w + (size_t)c0 * kConvTaps;   // [c][j], 16 contiguous values
    f4 rows[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) rows[k] = load4(wp + k * kConvTaps);   // channel c0 + k, taps 0..3
#pragma unroll
    for (int j = 0; j < kConvTaps; ++j) w[j] = f4{rows[0][j], rows[1][j], rows[2][j], rows[3][j]};
    b = a.bias ? load4((const TIn*)a.bias + c0) : f4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ f4 pre(f4 h0, f4 h1, f4 h2, f4 cur) const {
    return b + w[0] * h0 + w[1] * h1 + w[2] * h2 + w[3] * cur;
  }
};

template <typename TIn>
__global__ __launch_bounds__(256) void conv_fwd_kernel(ConvArgs a) {
  const int CG = a.C / 4;
  const int nstrips = (int)(((long long)a.T + kConvStrip - 1) / kConvStrip);
  const long long items = (long long)a.B * nstrips * CG;
  const TIn* u = (const TIn*)a.u;
  TIn* z = (TIn*)a.z;
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < items;
       it += (long long)gridDim.x * blockDim.x) {
    const int cg = (int)(it % CG);
    const long long pair = it / CG;
    const int b = (int)(pair / nstrips), t0 = (int)(pair % nstrips) * kConvStrip;
    const int c0 = cg * 4;
    ConvTaps<TIn> tp;
    tp.load(a, c0);
    const TIn* ub = u + (size_t)b * a.T * a.C + c0;
    f4 h[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int t = t0 - 3 + i;
      h[i] = t >= 0 ? load4(ub + (size_t)t * a.C) : f4{0.f, 0.f, 0.f, 0.f};
    }
    f4 cur[kConvStrip];
#pragma unroll
    for (int i = 0; i < kConvStrip; ++i) cur[i] = load4(ub + (size_t)min(t0 + i, a.T - 1) * a.C);   // clamped
    TIn* zb = z + (size_t)b * a.T * a.C + c0;
#pragma unroll
    for (int i = 0; i < kConvStrip; ++i) {
      const f4 x = tp.pre(i >= 3 ? cur[i - 3] : h[i], i >= 2 ? cur[i - 2] : h[i + 1], i >= 1 ? cur[i - 1] : h[2],
                          cur[i]);
      if (t0 + i < a.T) store4(zb + (size_t)(t0 + i) * a.C, x * sigmoid4(x));
    }
  }
}

// Backward: worker r of the R per channel group handles a contiguous run of
// (b, strip) pairs, p = b nstrips + strip in [r P / R, (r + 1) P / R), in
// order.  A strip at t0 needs u at t0 - 3 .. t0 + S + 2 and dz at t0 ..
// t0 + S + 2; the next strip of the same batch row shares six of those input
// rows and three dz rows, which stay in registers, so each row is read about
// once.  The worker keeps dw (four taps) and dbias of its four channels in
// registers; they go to ws[r][c * 4 + j] and ws[r][4 C + c], and a
// fixed-order column sum over the R rows gives dw and dbias.
template <typename TIn>
__global__ __launch_bounds__(256) void conv_bwd_kernel(ConvArgs a) {
  constexpr int S = kConvStripBwd;
  const int CG = a.C / 4;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= a.R * CG) return;
  const int cg = tid % CG, r = tid / CG;
  const int c0 = cg * 4;
  const int nstrips = (a.T + S - 1) / S;
  const long long P = (long long)a.B * nstrips;
  const long long p0 = r * P / a.R, p1 = (r + 1) * P / a.R;
  const TIn* u = (const TIn*)a.u;
  ConvTaps<TIn> tp;
  tp.load(a, c0);
  f4 dw[kConvTaps] = {}, db = {0.f, 0.f, 0.f, 0.f};
  f4 x[S + 6], g[S + 3];   // x[i]: u at t0 - 3 + i; g[i]: dz at t0 + i (zero outside [0, T))
  int prev_b = -1;
  for (long long p = p0; p < p1; ++p) {
    const int b = (int)(p / nstrips), t0 = (int)(p % nstrips) * S;
    const TIn* ub = u + (size_t)b * a.T * a.C + c0;
    const float* dzb = a.dz + (size_t)b * a.T * a.C + c0;
    const int keep_x = b == prev_b ? 6 : 0, keep_g = b == prev_b ? 3 : 0;
    if (b == prev_b) {
#pragma unroll
      for (int i = 0; i < 6; ++i) x[i] = x[i + S];
#pragma unroll
      for (int i = 0; i < 3; ++i) g[i] = g[i + S];
    }
#pragma unroll
    for (int i = 0; i < S + 6; ++i) {
      if (i < keep_x) continue;
      const int t = t0 - 3 + i;
      const f4 v = load4(ub + (size_t)min(max(t, 0), a.T - 1) * a.C);
      x[i] = (t < 0 || t >= a.T) ? f4{0.f, 0.f, 0.f, 0.f} : v;
    }
#pragma unroll
    for (int i = 0; i < S + 3; ++i) {
      if (i < keep_g) continue;
      const int t = t0 + i;
      const f4 v = load4(dzb + (size_t)min(t, a.T - 1) * a.C);
      g[i] = t >= a.T ? f4{0.f, 0.f, 0.f, 0.f} : v;
    }
    prev_b = b;
    // da at t0 + i (i < S + 3): x[i + 3] is the current input
    f4 da[S + 3];
#pragma unroll
    for (int i = 0; i < S + 3; ++i) {
      const f4 pa = tp.pre(x[i], x[i + 1], x[i + 2], x[i + 3]);
      const f4 sg = sigmoid4(pa);
      da[i] = g[i] * sg * (1.0f + pa * (1.0f - sg));
    }
    float* dub = a.du + (size_t)b * a.T * a.C + c0;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      if (t0 + i >= a.T) break;
      const f4 v = tp.w[3] * da[i] + tp.w[2] * da[i + 1] + tp.w[1] * da[i + 2] + tp.w[0] * da[i + 3];
      *(f4*)(dub + (size_t)(t0 + i) * a.C) = v;
#pragma unroll
      for (int j = 0; j < kConvTaps; ++j) dw[j] += da[i] * x[i + j];
      db += da[i];
    }
  }
  float* wsr = a.ws + (size_t)r * a.C * 5;
#pragma unroll
  for (int k = 0; k < 4; ++k) *(f4*)(wsr + (size_t)(c0 + k) * kConvTaps) = f4{dw[0][k], dw[1][k], dw[2][k], dw[3][k]};
  *(f4*)(wsr + (size_t)a.C * kConvTaps + c0) = db;
}

template <typename TIn>
hipError_t conv_fwd_t(const ConvArgs& a, hipStream_t stream) {
  const long long items = (long long)a.B * (((long long)a.T + kConvStrip - 1) / kConvStrip) * (a.C / 4);
  long long blocks = (items + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(conv_fwd_kernel<TIn>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename TIn>
hipError_t conv_bwd_t(const ConvArgs& a, hipStream_t stream) {
  const long long threads = (long long)a.R * (a.C / 4);
  hipLaunchKernelGGL(conv_bwd_kernel<TIn>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // columns: dw [C][4], then dbias [C]
  return launch_colsum(a.ws, a.R, a.C * 5, a.ws + (size_t)a.R * a.C * 5, a.dw, a.C * kConvTaps, a.dbias, stream);
}

}  // namespace

int conv_backward_workers(int B, int T, int C) {
  const long long npairs = (long long)B * (((long long)T + kConvStripBwd - 1) / kConvStripBwd);
  // about 262144 threads in all, each with at least four strips to carry rows across
  long long R = 262144 / (C / 4 > 0 ? C / 4 : 1);
  if (R > npairs / 4) R = npairs / 4;
  return R < 1 ? 1 : (int)R;
}

size_t conv_backward_workspace_floats(int B, int T, int C) {
  return ((size_t)conv_backward_workers(B, T, C) + kColsumRowBlocks) * (size_t)C * 5;
}

hipError_t launch_conv_forward(const ConvArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? conv_fwd_t<float>(a, stream) : conv_fwd_t<bf16_t>(a, stream);
}

hipError_t launch_conv_backward(const ConvArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? conv_bwd_t<float>(a, stream) : conv_bwd_t<bf16_t>(a, stream);
}

}  // namespace m2rnn

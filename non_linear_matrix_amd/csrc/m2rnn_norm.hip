// m2rnn_norm.hip -- output gate and RMSNorm after the scan's readout.
//
// After the readout the block multiplies y by the output gate g and applies
// RMSNorm over the token's d = N V features (slide "Most of the block can be
// computed before recurrence", paper Fig. 2).  The statistic and its backward
// are those of slide "Backup: RMSNormTP synchronizes per-token statistics"
// (paper App. C, Eqs. (26)-(33)), taken over the whole feature row on one GPU:
//     x = y g,   s = ((1/d) sum_j x_j^2 + eps)^{-1/2},   out_i = w_i x_i s
//     p = w dout,   r = sum_j p_j x_j,   dx = s p - (r s^3 / d) x
//     dy = dx g,   dg = dx y,   dw = sum over tokens of dout x s.
// The statistic couples all N heads of a token, which the scan spreads over
// many workgroups, so this is its own HBM-bound pass: one wave per token
// row, the row held in registers (C 16-byte chunks per lane, d <= 256 C <= 2048),
// sums by DPP within 16-lane rows and permlane swaps across rows.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

namespace {

// Sum over the 64 lanes; every lane gets the total.  v_permlane32_swap(x, x)
// returns the lower and upper 32-lane halves in the two results, and
// v_permlane16_swap(x, x) rows 0, 2 and rows 1, 3.
__device__ __forceinline__ float wave_sum(float x) {
  auto s32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                              false, false);
  x = __builtin_bit_cast(float, (uint32_t)s32[0]) + __builtin_bit_cast(float, (uint32_t)s32[1]);
  auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                              false, false);
  x = __builtin_bit_cast(float, (uint32_t)s16[0]) + __builtin_bit_cast(float, (uint32_t)s16[1]);
  return row_sum16(x);
}

__device__ __forceinline__ f4 load4(const float* p) { return *(const f4*)p; }
__device__ __forceinline__ f4 load4(const bf16_t* p) { return Vec4<bf16_t>::to_f4(*(const uint2*)p); }

__device__ __forceinline__ float dot4(f4 a, f4 b) { return (a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3]); }

constexpr int kWaves = 4;   // waves (token rows in flight) per workgroup

// Forward: wave `gw` of `nw` handles tokens gw, gw + nw, ...
template <typename TIn, int C>
__global__ __launch_bounds__(64 * kWaves) void norm_fwd_kernel(NormArgs a) {
  const int lane = threadIdx.x % 64;
  const long long nw = (long long)gridDim.x * kWaves;
  const int d = a.d;
  const TIn* g = (const TIn*)a.g;
  f4 wv[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = (c * 64 + lane) * 4;
    wv[c] = e < d ? load4((const TIn*)a.w + e) : f4{0.f, 0.f, 0.f, 0.f};
  }
  for (long long tok = (long long)blockIdx.x * kWaves + threadIdx.x / 64; tok < a.ntok; tok += nw) {
    const size_t row = (size_t)tok * d;
    f4 x[C];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (c * 64 + lane) * 4;
      x[c] = f4{0.f, 0.f, 0.f, 0.f};
      if (e < d) x[c] = load4(a.y + row + e) * load4(g + row + e);
      ss += dot4(x[c], x[c]);
    }
    const float s = __builtin_amdgcn_rsqf(wave_sum(ss) / (float)d + a.eps);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (c * 64 + lane) * 4;
      if (e < d) *(f4*)(a.out + row + e) = wv[c] * x[c] * s;
    }
    if (a.rstd && lane == 0) a.rstd[tok] = s;
  }
}

// Backward: as the forward, one wave per token row, plus the wave's dw
// partial in registers; the workgroup sums its waves' partials into
// ws[blockIdx.x][d] in a fixed order.
template <typename TIn, int C>
__global__ __launch_bounds__(64 * kWaves) void norm_bwd_kernel(NormArgs a) {
  __shared__ f4 part[kWaves][C * 64];
  const int lane = threadIdx.x % 64, wv_id = threadIdx.x / 64;
  const long long nw = (long long)gridDim.x * kWaves;
  const int d = a.d;
  const TIn* g = (const TIn*)a.g;
  const float inv_d = 1.0f / (float)d;
  f4 wv[C], dwp[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = (c * 64 + lane) * 4;
    wv[c] = e < d ? load4((const TIn*)a.w + e) : f4{0.f, 0.f, 0.f, 0.f};
    dwp[c] = f4{0.f, 0.f, 0.f, 0.f};
  }
  for (long long tok = (long long)blockIdx.x * kWaves + wv_id; tok < a.ntok; tok += nw) {
    const size_t row = (size_t)tok * d;
    f4 yv[C], gv[C], dov[C];
    float ss = 0.f, r = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (c * 64 + lane) * 4;
      yv[c] = gv[c] = dov[c] = f4{0.f, 0.f, 0.f, 0.f};
      if (e < d) {
        yv[c] = load4(a.y + row + e);
        gv[c] = load4(g + row + e);
        dov[c] = load4(a.dout + row + e);
      }
      const f4 x = yv[c] * gv[c];
      ss += dot4(x, x);
      r += dot4(wv[c] * dov[c], x);
    }
    ss = wave_sum(ss);
    r = wave_sum(r);
    const float s = __builtin_amdgcn_rsqf(ss * inv_d + a.eps);
    const float k = r * s * s * s * inv_d;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (c * 64 + lane) * 4;
      const f4 x = yv[c] * gv[c];
      const f4 dx = s * (wv[c] * dov[c]) - k * x;
      dwp[c] += dov[c] * x * s;
      if (e < d) {
        *(f4*)(a.dy + row + e) = dx * gv[c];
        *(f4*)(a.dg + row + e) = dx * yv[c];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) part[wv_id][c * 64 + lane] = dwp[c];
  __syncthreads();
  for (int u = threadIdx.x; u < C * 64; u += 64 * kWaves) {
    f4 acc = part[0][u];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) acc += part[v][u];
    const int e = u * 4;
    if (e < d) *(f4*)(a.ws + (size_t)blockIdx.x * d + e) = acc;
  }
}

int chunks_for(int d) {
  const int c = (d + 255) / 256;
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 8;
}

template <typename TIn>
hipError_t norm_fwd_t(const NormArgs& a, hipStream_t stream) {
  long long wg = (a.ntok + kWaves - 1) / kWaves;
  if (wg > 8192) wg = 8192;
  const dim3 grid((unsigned)wg), block(64 * kWaves);
  switch (chunks_for(a.d)) {
    case 1: hipLaunchKernelGGL((norm_fwd_kernel<TIn, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((norm_fwd_kernel<TIn, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((norm_fwd_kernel<TIn, 4>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((norm_fwd_kernel<TIn, 8>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

template <typename TIn>
hipError_t norm_bwd_t(const NormArgs& a, hipStream_t stream) {
  const int nwg = norm_backward_groups(a.ntok, a.d);
  const dim3 grid((unsigned)nwg), block(64 * kWaves);
  switch (chunks_for(a.d)) {
    case 1: hipLaunchKernelGGL((norm_bwd_kernel<TIn, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((norm_bwd_kernel<TIn, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((norm_bwd_kernel<TIn, 4>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((norm_bwd_kernel<TIn, 8>), grid, block, 0, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_colsum(a.ws, nwg, a.d, a.ws + (size_t)nwg * a.d, a.dw, a.d, nullptr, stream);
}

}  // namespace

int norm_backward_groups(long long ntok, int d) {
  (void)d;
  long long wg = (ntok + kWaves - 1) / kWaves;
  if (wg > kNormMaxGroups) wg = kNormMaxGroups;
  return wg < 1 ? 1 : (int)wg;
}

size_t norm_backward_workspace_floats(long long ntok, int d) {
  return ((size_t)norm_backward_groups(ntok, d) + kColsumRowBlocks) * (size_t)d;
}

hipError_t launch_norm_forward(const NormArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? norm_fwd_t<float>(a, stream) : norm_fwd_t<bf16_t>(a, stream);
}

hipError_t launch_norm_backward(const NormArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? norm_bwd_t<float>(a, stream) : norm_bwd_t<bf16_t>(a, stream);
}

}  // namespace m2rnn

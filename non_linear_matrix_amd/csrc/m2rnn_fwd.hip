// m2rnn_fwd.hip -- persistent forward scan of the M2RNN recurrence on gfx950.
//
// Method: M2RNN paper-discussion slides (reading of arXiv:2603.14360v2),
// slide "Write, transform, retain, and read a matrix state" (paper
// Eqs. (10)-(12)):  Z_t = tanh(H_{t-1} W + k_t v_t^T),
// H_t = f_t H_{t-1} + (1 - f_t) Z_t,  y_t = H_t^T q_t + w_r (.) v_t,  H_0 = 0;
// q_t, k_t shared by the N value heads (slide "Shared queries and keys buy
// more recurrent capacity", paper Alg. 1).  The slides' kernel keeps H and W
// on chip and scans time sequentially per (batch, head) (slide "Efficient
// tiles do not remove the sequential dependency", paper Sec. 4.1); this
// kernel does the same with an MI355X-specific register layout:
//
//  * one wave64 owns one (b, n) head for the whole sequence; its 64 x 16 state
//    sits in four MFMA accumulators (see m2rnn_device.h);
//  * H_{t-1} W is one v_mfma_f32_16x16x32_bf16 per row tile: W^T in the A
//    operand (resident), hi/lo bf16 split of the fp32 state in the B operand
//    (fp32 inputs add a second MFMA for the low half of W);
//  * k v^T, tanh, the gate and the readout products are fused per lane;
//    the readout sum over the 64 rows is an in-register sum over the four
//    tiles plus a 16-lane DPP reduction;
//  * a workgroup of NW waves covers NW heads of one batch row and streams
//    q, k, v, f for TC steps at a time from HBM into LDS, double-buffered,
//    prefetching chunk c+1 into registers while chunk c is computed; y is
//    staged in LDS and written back as contiguous NW*16-float rows.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

template <int NW, int TC>
struct FwdSmem {
  // per buffer: K_s[TC][64], Q_s[TC][64], V_s[TC][NW][16], F_s[TC][NW][4]
  static constexpr int kPerStep = 64 + 64 + NW * 16 + NW * 4;
  static constexpr int kBuf = TC * kPerStep;
  static constexpr int kY = TC * NW * 16;
  static constexpr int kFloats = 2 * kBuf + kY;
  static constexpr int kBytes = kFloats * 4;
};

template <typename TIn, int NW, int TC>
struct FwdStager {
  typedef typename Vec4<TIn>::raw raw;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kQK = (2 * TC * 16 + kThreads - 1) / kThreads;  // 4-vectors of q and k
  static constexpr int kV = (TC * NW * 4 + kThreads - 1) / kThreads;   // 4-vectors of v
  raw qk[kQK];
  raw vv[kV];
  float ff;

  __device__ void load(const FwdArgs& a, int b, int n0, int t0, int tid) {
#pragma unroll
    for (int r = 0; r < kQK; ++r) {
      int u = tid + r * kThreads;           // [0, 2*TC*16)
      int which = u / (TC * 16);            // 0: q, 1: k
      int t = (u / 16) % TC, e0 = (u % 16) * 4;
      qk[r] = Vec4<TIn>::zero();
      if (u < 2 * TC * 16 && t0 + t < a.T) {
        const TIn* src = (const TIn*)(which ? a.k : a.q);
        qk[r] = Vec4<TIn>::load(src + ((size_t)b * a.T + t0 + t) * 64 + e0);
      }
    }
#pragma unroll
    for (int r = 0; r < kV; ++r) {
      int u = tid + r * kThreads;           // [0, TC*NW*4)
      int t = u / (NW * 4), h = (u / 4) % NW, c4 = u % 4;
      vv[r] = Vec4<TIn>::zero();
      if (u < TC * NW * 4 && t0 + t < a.T && n0 + h < a.N)
        vv[r] = Vec4<TIn>::load((const TIn*)a.v + (((size_t)b * a.T + t0 + t) * a.N + n0 + h) * 16 + 4 * c4);
    }
    ff = 1.0f;
    {
      int t = tid / NW, h = tid % NW;
      if (tid < TC * NW && t0 + t < a.T && n0 + h < a.N)
        ff = to_f32(((const TIn*)a.f)[((size_t)b * a.T + t0 + t) * a.N + n0 + h]);
    }
  }

  __device__ void store(float* buf, int tid) const {
    float* K_s = buf;
    float* Q_s = buf + TC * 64;
    float* V_s = buf + 2 * TC * 64;
    float* F_s = V_s + TC * NW * 16;
#pragma unroll
    for (int r = 0; r < kQK; ++r) {
      int u = tid + r * kThreads;
      if (u < 2 * TC * 16) {
        int which = u / (TC * 16);
        int t = (u / 16) % TC, e0 = (u % 16) * 4;
        f4 x = Vec4<TIn>::to_f4(qk[r]);
        // element e = 16 j + m goes to [t][m][j]: a lane with column m reads
        // its four tiles' values as one 16-byte word.
        float* dst = (which ? K_s : Q_s) + t * 64;
        float s = which ? kScale : kInvScale;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int e = e0 + i;
          dst[(e % 16) * 4 + e / 16] = x[i] * s;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kV; ++r) {
      int u = tid + r * kThreads;
      if (u < TC * NW * 4) *(f4*)(V_s + u * 4) = Vec4<TIn>::to_f4(vv[r]);
    }
    if (tid < TC * NW) {
      float g = 1.0f - ff;
      *(f4*)(F_s + tid * 4) = f4{ff, kScale * g, -2.0f * kScale * g, 0.0f};
    }
  }
};

template <typename TIn, int NW, int TC>
__global__ __launch_bounds__(64 * NW) void m2rnn_fwd_kernel(FwdArgs a) {
  typedef FwdSmem<NW, TC> Sm;
  extern __shared__ float smem[];
  float* ystage = smem + 2 * Sm::kBuf;

  const int tid = threadIdx.x;
  const int w = tid / 64, lane = tid % 64, g = lane / 16, m = lane % 16;
  const int ngroups = (a.N + NW - 1) / NW;
  const int b = blockIdx.x / ngroups;
  const int n0 = (blockIdx.x % ngroups) * NW;
  const int n = n0 + w;
  const bool live = n < a.N;

  // Resident W^T operand.  bf16 inputs: slot s of lane group g multiplies
  // state row v = 4g + (s & 3) (hi half in slots 0..3, lo half in 4..7).
  // fp32 inputs: instruction r of the four 16x16x4 MFMAs multiplies row 4g + r.
  WOperand<TIn> Aw;
  Aw.load(live ? (const TIn*)a.W + (size_t)n * 256 : nullptr, g, m);
  f4 wr4 = {0.f, 0.f, 0.f, 0.f};
  if (live) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wr4[i] = to_f32(((const TIn*)a.wr)[(size_t)n * 16 + 4 * g + i]);
  }

  f4 P[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) P[j] = f4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (a.T + TC - 1) / TC;
  FwdStager<TIn, NW, TC> st;
  st.load(a, b, n0, 0, tid);
  st.store(smem, tid);
  __syncthreads();

  int next_ck = a.H_ckpt ? 0 : a.T;  // next step whose incoming state is checkpointed
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * TC;
    const bool more = c + 1 < nchunks;
    if (more) st.load(a, b, n0, t0 + TC, tid);

    const float* buf = smem + (c & 1) * Sm::kBuf;
    const float* K_s = buf;
    const float* Q_s = buf + TC * 64;
    const float* V_s = buf + 2 * TC * 64;
    const float* F_s = V_s + TC * NW * 16;
    const int steps = min(TC, a.T - t0);
    if (live) {
      for (int tt = 0; tt < steps; ++tt) {
        const int t = t0 + tt;
        if (t == next_ck) {
          float* dst = a.H_ckpt + (((size_t)b * a.N + n) * a.nck + t / a.ckpt_every) * 1024;
          next_ck += a.ckpt_every;
#pragma unroll
          for (int j = 0; j < 4; ++j) *(f4*)(dst + (16 * j + m) * 16 + 4 * g) = P[j] * kInvScale;
        }
        const f4 kq = *(const f4*)(K_s + tt * 64 + m * 4);   // c k[16j+m]
        const f4 qq = *(const f4*)(Q_s + tt * 64 + m * 4);   // q[16j+m] / c
        const f4 vv = *(const f4*)(V_s + (tt * NW + w) * 16 + 4 * g);
        const f4 fc = *(const f4*)(F_s + (tt * NW + w) * 4); // f, c(1-f), -2c(1-f)
        f4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f4 D = Aw.times_state(P[j]);                     // c (H W)^T tile
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = fmaf(kq[j], vv[i], D[i]);             // c * (H W + k v^T)
            const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x) + 1.0f);  // (1 - tanh)/2
            const float h = fmaf(fc[0], P[j][i], fc[1]);          // f P + c (1 - f)
            P[j][i] = fmaf(fc[2], r, h);                          // f P + c (1 - f) tanh
            p[i] = fmaf(P[j][i], qq[j], p[i]);
          }
        }
        f4 y4;
#pragma unroll
        for (int i = 0; i < 4; ++i) y4[i] = fmaf(wr4[i], vv[i], row_sum16(p[i]));
        if (m == 0) *(f4*)(ystage + (tt * NW + w) * 16 + 4 * g) = y4;
      }
    }
    __syncthreads();
    // y rows of this chunk: [t][n0 .. n0+NW)[16], contiguous per t
#pragma unroll
    for (int r = 0; r < (TC * NW * 4 + 64 * NW - 1) / (64 * NW); ++r) {
      int u = tid + r * 64 * NW;
      int tt = u / (NW * 4), h = (u / 4) % NW, c4 = u % 4;
      if (u < TC * NW * 4 && tt < steps && n0 + h < a.N)
        *(f4*)(a.y + (((size_t)b * a.T + t0 + tt) * a.N + n0 + h) * 16 + 4 * c4) = *(const f4*)(ystage + u * 4);
    }
    if (more) st.store(smem + ((c + 1) & 1) * Sm::kBuf, tid);
    __syncthreads();
  }

  if (live) {
    float* dst = a.H_T + ((size_t)b * a.N + n) * 1024;
#pragma unroll
    for (int j = 0; j < 4; ++j) *(f4*)(dst + (16 * j + m) * 16 + 4 * g) = P[j] * kInvScale;
  }
}

template <typename TIn, int NW>
static hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  constexpr int TC = 32;
  typedef FwdSmem<NW, TC> Sm;
  static_assert(Sm::kBytes <= 64 * 1024, "forward LDS budget");
  const int ngroups = (a.N + NW - 1) / NW;
  dim3 grid((unsigned)(a.B * ngroups)), block(64 * NW);
  hipLaunchKernelGGL((m2rnn_fwd_kernel<TIn, NW, TC>), grid, block, Sm::kBytes, stream, a);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t dispatch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.N >= 4) return launch_fwd<TIn, 4>(a, stream);
  if (a.N >= 2) return launch_fwd<TIn, 2>(a, stream);
  return launch_fwd<TIn, 1>(a, stream);
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.0f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? dispatch_fwd<float>(a, stream) : dispatch_fwd<bf16_t>(a, stream);
}

}  // namespace m2rnn

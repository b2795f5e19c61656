// m2rnn_bwd.hip -- backward scan (BPTT) of the M2RNN recurrence on gfx950.
//
// Method: M2RNN paper-discussion slides (reading of arXiv:2603.14360v2),
// slide "Backup: the recurrent gradient needs both paths": with u_t = dL/dy_t
// and C_t the gradient reaching H_t from later steps,
//     R_t = C_t + q_t u_t^T,   D_t = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t),
//     C_{t-1} = f_t R_t + D_t W^T,   dL/df_t = <R_t, H_{t-1} - Z_t>,
//     dL/dW = sum_t H_{t-1}^T D_t,
// and, by the chain rule on the forward equations (slide "Write, transform,
// retain, and read a matrix state", paper Eqs. (10)-(12)),
//     dL/dk_t = D_t v_t,  dL/dv_t = D_t^T k_t + w_r (.) u_t,
//     dL/dq_t = H_t u_t,  dL/dw_r = sum_t u_t (.) v_t,
// with dq, dk summed over the heads sharing q_t, k_t.  The slides' own kernel
// recomputes the trajectory and caches every state in HBM (slide "Efficient
// tiles do not remove the sequential dependency"); this one keeps the caches
// on chip instead:
//
//  * one wave64 owns one 16-row tile of one (b, n) head (rows of H never mix
//    in the recurrence; only the reductions couple them), so a head is four
//    waves of one workgroup and a workgroup holds HPW heads of a batch row;
//  * the forward stored H every `ckpt_every` steps.  Per checkpoint chunk,
//    level 1 replays the chunk and writes a sub-checkpoint every kSub steps
//    to the workspace; level 2 replays each sub-chunk (latest first) keeping
//    H_{t-1} and Z_t of its kSub steps in registers, then the reverse sweep
//    walks those steps back;
//  * C_{t-1}^T = f R^T + W D^T is one v_mfma_f32_16x16x32_bf16 per step (W in
//    the A operand, hi/lo split of D^T in B, f R^T as the accumulator input;
//    four exact fp32 MFMAs for fp32 inputs), in the same transposed frame as
//    the forward, so C stays in registers;
//  * dW needs a contraction over the rows, which live on lanes: each step the
//    wave writes its H_{t-1} and D tiles to LDS and reads them back in MFMA
//    operand layout for four exact v_mfma_f32_16x16x4_f32, accumulated in
//    registers over the whole sequence;
//  * per-step sums over a head's rows (df, dv) and over the heads of the
//    workgroup (dq, dk) go through LDS after every sub-chunk; the sums over
//    workgroups (dq, dk) and batch rows (dW, dw_r) are a second, fixed-order
//    reduction kernel.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

constexpr int kSub = 8;  // steps kept in registers by the level-2 replay

template <int HPW>
struct BwdCfg {
  static constexpr int NWAVES = HPW * 4;
  static constexpr int NT = 64 * NWAVES;
  // per staged step: K_s[64] (c k), Q_s[64] (q), V_s[HPW][16], F_s[HPW][4], U_s[HPW][16]
  static constexpr int kStep = 128 + HPW * 36;
  static constexpr int kBuf = kSub * kStep;
  static constexpr int kXpose = NWAVES * 512;          // per wave: H_{t-1} tile, D tile
  static constexpr int kDf = kSub * HPW * 4;           // [s][h][tile]
  static constexpr int kDv = kSub * HPW * 4 * 16;      // [s][h][tile][16]
  static constexpr int kDqk = kSub * HPW * 2 * 64;     // [s][h][dq|dk][64]
  static constexpr int kFloats = 2 * kBuf + kXpose + kDf + kDv + kDqk;
  static constexpr int kBytes = kFloats * 4;
};

// Staging of one sub-chunk (up to kSub steps starting at t0) for HPW heads.
template <typename TIn, int HPW, int NT>
struct BwdStager {
  typedef typename Vec4<TIn>::raw raw;
  static constexpr int kQK = (2 * kSub * 16 + NT - 1) / NT;
  static constexpr int kV = (kSub * HPW * 4 + NT - 1) / NT;
  raw qk[kQK];
  raw vv[kV];
  f4 uu[kV];
  float ff;

  __device__ void load(const BwdArgs& a, int b, int n0, int t0, int len, int tid) {
#pragma unroll
    for (int r = 0; r < kQK; ++r) {
      int u = tid + r * NT;
      int which = u / (kSub * 16);
      int t = (u / 16) % kSub, e0 = (u % 16) * 4;
      qk[r] = Vec4<TIn>::zero();
      if (u < 2 * kSub * 16 && t < len) {
        const TIn* src = (const TIn*)(which ? a.k : a.q);
        qk[r] = Vec4<TIn>::load(src + ((size_t)b * a.T + t0 + t) * 64 + e0);
      }
    }
#pragma unroll
    for (int r = 0; r < kV; ++r) {
      int u = tid + r * NT;
      int t = u / (HPW * 4), h = (u / 4) % HPW, c4 = u % 4;
      vv[r] = Vec4<TIn>::zero();
      uu[r] = f4{0.f, 0.f, 0.f, 0.f};
      if (u < kSub * HPW * 4 && t < len && n0 + h < a.N) {
        const size_t off = (((size_t)b * a.T + t0 + t) * a.N + n0 + h) * 16 + 4 * c4;
        vv[r] = Vec4<TIn>::load((const TIn*)a.v + off);
        uu[r] = *(const f4*)(a.dy + off);
      }
    }
    ff = 1.0f;
    {
      int t = tid / HPW, h = tid % HPW;
      if (tid < kSub * HPW && t < len && n0 + h < a.N)
        ff = to_f32(((const TIn*)a.f)[((size_t)b * a.T + t0 + t) * a.N + n0 + h]);
    }
  }

  __device__ void store(float* buf, int tid) const {
    float* K_s = buf;
    float* Q_s = K_s + kSub * 64;
    float* V_s = Q_s + kSub * 64;
    float* F_s = V_s + kSub * HPW * 16;
    float* U_s = F_s + kSub * HPW * 4;
#pragma unroll
    for (int r = 0; r < kQK; ++r) {
      int u = tid + r * NT;
      if (u < 2 * kSub * 16) {
        int which = u / (kSub * 16);
        int t = (u / 16) % kSub, e0 = (u % 16) * 4;
        f4 x = Vec4<TIn>::to_f4(qk[r]);
        if (which) x *= kScale;
        *(f4*)((which ? K_s : Q_s) + t * 64 + e0) = x;
      }
    }
#pragma unroll
    for (int r = 0; r < kV; ++r) {
      int u = tid + r * NT;
      if (u < kSub * HPW * 4) {
        *(f4*)(V_s + u * 4) = Vec4<TIn>::to_f4(vv[r]);
        *(f4*)(U_s + u * 4) = uu[r];
      }
    }
    if (tid < kSub * HPW) {
      float gg = 1.0f - ff;
      *(f4*)(F_s + tid * 4) = f4{ff, kScale * gg, -2.0f * kScale * gg, gg};
    }
  }
};

// Accumulator-input variant of the contraction used by the C update:
// returns (W D^T)^T + cin in the transposed frame, i.e. A = W (not W^T).
template <typename TIn> struct WBackOperand;
template <> struct WBackOperand<bf16_t> {
  bf16x8 a;
  __device__ void load(const bf16_t* Wn, int g, int m) {
    float w[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x = Wn ? to_f32(Wn[m * 16 + 4 * g + s]) : 0.0f;   // W[v = m][v' = 4g + s]
      w[s] = w[s + 4] = x;
    }
    a = pack8(w);
  }
  __device__ f4 apply(f4 d, f4 cin) const { return mfma_bf16(a, split_operand(d), cin); }
};
template <> struct WBackOperand<float> {
  float a[4];
  __device__ void load(const float* Wn, int g, int m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = Wn ? Wn[m * 16 + 4 * g + r] : 0.0f;
  }
  __device__ f4 apply(f4 d, f4 cin) const {
#pragma unroll
    for (int r = 0; r < 4; ++r) cin = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], d[r], cin, 0, 0, 0);
    return cin;
  }
};

__device__ __forceinline__ float sum_lane_groups(float x) {  // over lanes m, m+16, m+32, m+48
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// One forward step of one tile (no readout): returns r = (1 - tanh)/2 and
// updates P in place.
template <typename TIn>
__device__ __forceinline__ f4 fwd_tile_step(const WOperand<TIn>& Aw, f4& P, float ck, f4 vv, f4 fc) {
  f4 x = Aw.times_state(P);
  f4 r, hg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = fmaf(ck, vv[i], x[i]);
    hg[i] = fmaf(fc[0], P[i], fc[1]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x[i]) + 1.0f);
#pragma unroll
  for (int i = 0; i < 4; ++i) P[i] = fmaf(fc[2], r[i], hg[i]);
  return r;
}

template <typename TIn, int HPW>
__global__ __launch_bounds__(256 * HPW) void m2rnn_bwd_kernel(BwdArgs a) {
  typedef BwdCfg<HPW> Cfg;
  constexpr int NT = Cfg::NT;
  extern __shared__ float smem[];
  float* xpose = smem + 2 * Cfg::kBuf;
  float* dfbuf = xpose + Cfg::kXpose;
  float* dvbuf = dfbuf + Cfg::kDf;
  float* dqkbuf = dvbuf + Cfg::kDv;

  const int tid = threadIdx.x;
  // wave-uniform indices live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, g = lane / 16, m = lane % 16;
  const int hw = w / 4, j = w % 4;               // head in group, row tile
  const int ngroups = (a.N + HPW - 1) / HPW;
  const int b = blockIdx.x / ngroups;
  const int grp = blockIdx.x % ngroups;
  const int n0 = grp * HPW;
  const int n = n0 + hw;
  const bool live = n < a.N;
  const int kk = 16 * j + m;                      // this lane's state row
  float* xp = xpose + w * 512;
  const size_t head = (size_t)b * a.N + n;
  // stored states H at t = s * L (s = 0 .. ns-1), L = a.ckpt_every <= kSub
  const int L = a.ckpt_every, ns = a.nck;
  const float* Hs = a.H_ckpt + head * (size_t)ns * 1024 + kk * 16 + 4 * g;

  WOperand<TIn> Af;
  Af.load(live ? (const TIn*)a.W + (size_t)n * 256 : nullptr, g, m);
  WBackOperand<TIn> Ab;
  Ab.load(live ? (const TIn*)a.W + (size_t)n * 256 : nullptr, g, m);

  // C in the transposed frame: lane (g, m), register i = C[kk][4g + i]
  f4 C = {0.f, 0.f, 0.f, 0.f};
  if (live && a.dH_T) C = *(const f4*)(a.dH_T + head * 1024 + kk * 16 + 4 * g);
  f4 dW = {0.f, 0.f, 0.f, 0.f};   // lane (g, m), register i: c * dW[4g + i][m] partial
  f4 dwr = {0.f, 0.f, 0.f, 0.f};

  BwdStager<TIn, HPW, NT> st;
  {
    const int t0 = (ns - 1) * L;
    st.load(a, b, n0, t0, min(L, a.T - t0), tid);
    st.store(smem, tid);
  }
  f4 Pnext = {0.f, 0.f, 0.f, 0.f};
  if (live) Pnext = *(const f4*)(Hs + (size_t)(ns - 1) * 1024) * kScale;
  __syncthreads();

  for (int sb = ns - 1, it = 0; sb >= 0; --sb, ++it) {
    const int t0 = sb * L, len = min(L, a.T - t0);
    const bool more = sb > 0;
    f4 P = Pnext;
    if (more) {
      st.load(a, b, n0, t0 - L, L, tid);
      if (live) Pnext = *(const f4*)(Hs + (size_t)(sb - 1) * 1024) * kScale;
    }
    const float* buf = smem + (it & 1) * Cfg::kBuf;
    const float* K_s = buf;
    const float* Q_s = K_s + kSub * 64;
    const float* V_s = Q_s + kSub * 64;
    const float* F_s = V_s + kSub * HPW * 16;
    const float* U_s = F_s + kSub * HPW * 4;

    if (live) {
      // replay the sub-chunk keeping H_{t-1} and Z_t on chip
      f4 Pp[kSub], Z[kSub];
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        if (s < len) {
          const f4 vv = *(const f4*)(V_s + (s * HPW + hw) * 16 + 4 * g);
          const f4 fc = *(const f4*)(F_s + (s * HPW + hw) * 4);
          const f4 uu = *(const f4*)(U_s + (s * HPW + hw) * 16 + 4 * g);
          Pp[s] = P;
          const f4 r = fwd_tile_step<TIn>(Af, P, K_s[s * 64 + kk], vv, fc);
#pragma unroll
          for (int i = 0; i < 4; ++i) Z[s][i] = fmaf(-2.0f, r[i], 1.0f);
          // dq_t[kk] (this head) = sum_v H_t[kk][v] u_t[v] = (1/c) sum_v P u
          float dq = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) dq = fmaf(P[i], uu[i], dq);
          dq = sum_lane_groups(dq);
          if (g == 0) dqkbuf[(s * HPW + hw) * 128 + kk] = dq * kInvScale;
        }
        __builtin_amdgcn_sched_barrier(0);   // keep each step's loads in its step
      }
      // reverse sweep over the sub-chunk
#pragma unroll
      for (int s = kSub - 1; s >= 0; --s) {
        if (s < len) {
          const f4 vv = *(const f4*)(V_s + (s * HPW + hw) * 16 + 4 * g);
          const f4 fc = *(const f4*)(F_s + (s * HPW + hw) * 4);   // f, c(1-f), -2c(1-f), 1-f
          const f4 uu = *(const f4*)(U_s + (s * HPW + hw) * 16 + 4 * g);
          const float qv = Q_s[s * 64 + kk];
          const float ckv = K_s[s * 64 + kk];                      // c k[kk]
          f4 R, D, fR;
          float dfp = 0.f, dk = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            R[i] = fmaf(qv, uu[i], C[i]);                            // R = C + q u^T
            const float gz = fc[3] * Z[s][i];
            D[i] = R[i] * fmaf(-gz, Z[s][i], fc[3]);                 // (1-f) R (1 - Z^2)
            dfp = fmaf(R[i], fmaf(Pp[s][i], kInvScale, -Z[s][i]), dfp);   // <R, H_{t-1} - Z>
            fR[i] = fc[0] * R[i];
            dk = fmaf(D[i], vv[i], dk);
            dwr[i] = fmaf(uu[i], vv[i], dwr[i]);
          }
          C = Ab.apply(D, fR);                                       // C_{t-1} = f R + D W^T
          // dk_t[kk] (this head) = sum_v' D[kk][v'] v[v']
          dk = sum_lane_groups(dk);
          if (g == 0) dqkbuf[(s * HPW + hw) * 128 + 64 + kk] = dk;
          // dv_t[v'] partial over this tile's rows: sum_kk D[kk][v'] (c k[kk])
          f4 dvp;
#pragma unroll
          for (int i = 0; i < 4; ++i) dvp[i] = row_sum16(D[i] * ckv);
          if (m == 0) *(f4*)(dvbuf + ((s * HPW + hw) * 4 + j) * 16 + 4 * g) = dvp;
          // df_t partial over this tile
          dfp = sum_lane_groups(row_sum16(dfp));
          if (lane == 0) dfbuf[(s * HPW + hw) * 4 + j] = dfp;
          // dW += H_{t-1}^T D via LDS transpose + four exact fp32 MFMAs
          *(f4*)(xp + m * 16 + 4 * g) = Pp[s];
          *(f4*)(xp + 256 + m * 16 + 4 * g) = D;
          wave_lds_fence();
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float av = xp[(4 * r + g) * 16 + m];        // c H_{t-1}[4r+g][v = m]
            const float bv = xp[256 + (4 * r + g) * 16 + m];  // D[4r+g][v' = m]
            dW = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, dW, 0, 0, 0);
          }
          wave_lds_fence();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    // df[b][t][n] = sum over the four tiles
    if (tid < len * HPW) {
      const int s = tid / HPW, hh = tid % HPW;
      if (n0 + hh < a.N) {
        const float* d4 = dfbuf + (s * HPW + hh) * 4;
        a.df[((size_t)b * a.T + t0 + s) * a.N + n0 + hh] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      }
    }
    // dv[b][t][n][:] = (1/c) sum over tiles + w_r * u
    for (int u = tid; u < len * HPW * 4; u += NT) {
      const int s = u / (HPW * 4), hh = (u / 4) % HPW, c4 = u % 4;
      if (n0 + hh < a.N) {
        const float* d = dvbuf + ((s * HPW + hh) * 4) * 16 + 4 * c4;
        f4 acc = (*(const f4*)d + *(const f4*)(d + 16)) + (*(const f4*)(d + 32) + *(const f4*)(d + 48));
        const f4 uu = *(const f4*)(U_s + (s * HPW + hh) * 16 + 4 * c4);
        const TIn* wrp = (const TIn*)a.wr + (size_t)(n0 + hh) * 16 + 4 * c4;
        f4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = fmaf(to_f32(wrp[i]), uu[i], acc[i] * kInvScale);
        *(f4*)(a.dv + (((size_t)b * a.T + t0 + s) * a.N + n0 + hh) * 16 + 4 * c4) = out;
      }
    }
    // dq, dk partials of this workgroup's heads -> workspace [b][grp][t][dq|dk][64]
    for (int u = tid; u < len * 32; u += NT) {
      const int s = u / 32, e = (u % 32) * 4;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int hh = 0; hh < HPW; ++hh)
        if (n0 + hh < a.N) acc += *(const f4*)(dqkbuf + (s * HPW + hh) * 128 + e);
      *(f4*)(a.ws_dqk + (((size_t)b * ngroups + grp) * a.T + t0 + s) * 128 + e) = acc;
    }
    if (more) st.store(smem + ((it + 1) & 1) * Cfg::kBuf, tid);
    __syncthreads();
  }

  if (live) {
    float* dst = a.ws_dW + (head * 4 + j) * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * g + i) * 16 + m] = dW[i] * kInvScale;
    if (j == 0 && m == 0) *(f4*)(a.ws_dwr + head * 16 + 4 * g) = dwr;
  }
}

// Fixed-order sums over workgroups (dq, dk), batch rows and row tiles (dW),
// and batch rows (dw_r).
__global__ void m2rnn_bwd_reduce_kernel(BwdArgs a) {
  const size_t nqk = (size_t)a.B * a.T * 32;   // float4 groups of dq and dk
  const size_t nW = (size_t)a.N * 64;          // float4 groups of dW
  const size_t nwr = (size_t)a.N * 4;
  const size_t total = nqk + nW + nwr;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    if (u < nqk) {
      const size_t bt = u / 32;
      const int e = (int)(u % 32) * 4;
      const size_t b = bt / a.T, t = bt % a.T;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int gp = 0; gp < a.ngroups; ++gp) acc += *(const f4*)(a.ws_dqk + ((b * a.ngroups + gp) * a.T + t) * 128 + e);
      float* dst = e < 64 ? a.dq + bt * 64 + e : a.dk + bt * 64 + (e - 64);
      *(f4*)dst = acc;
    } else if (u < nqk + nW) {
      const size_t v = u - nqk;
      const size_t n = v / 64;
      const int e = (int)(v % 64) * 4;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int b = 0; b < a.B; ++b)
        for (int jt = 0; jt < 4; ++jt) acc += *(const f4*)(a.ws_dW + (((size_t)b * a.N + n) * 4 + jt) * 256 + e);
      *(f4*)(a.dW + n * 256 + e) = acc;
    } else {
      const size_t v = u - nqk - nW;
      const size_t n = v / 4;
      const int e = (int)(v % 4) * 4;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int b = 0; b < a.B; ++b) acc += *(const f4*)(a.ws_dwr + ((size_t)b * a.N + n) * 16 + e);
      *(f4*)(a.dw_r + n * 16 + e) = acc;
    }
  }
}

constexpr int kBwdHPW = 2;

size_t backward_workspace_floats(int B, int T, int N, int ckpt_every, size_t* off_dense, size_t* off_dqk,
                                 size_t* off_dW, size_t* off_dwr, int* ngroups) {
  const int ng = (N + kBwdHPW - 1) / kBwdHPW;
  auto up = [](size_t x) { return (x + 63) & ~(size_t)63; };   // 256-byte aligned regions
  size_t o = 0;
  *off_dense = o;
  if (ckpt_every > kSub) o += up((size_t)B * N * ((T + kSub - 1) / kSub) * 1024);
  *off_dqk = o;  o += up((size_t)B * ng * T * 128);
  *off_dW = o;   o += up((size_t)B * N * 4 * 256);
  *off_dwr = o;  o += up((size_t)B * N * 16);
  *ngroups = ng;
  return o;
}

template <typename TIn>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  typedef BwdCfg<kBwdHPW> Cfg;
  static_assert(Cfg::kBytes <= 64 * 1024, "backward LDS budget");
  dim3 grid((unsigned)(a.B * a.ngroups)), block(Cfg::NT);
  hipLaunchKernelGGL((m2rnn_bwd_kernel<TIn, kBwdHPW>), grid, block, Cfg::kBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)a.B * a.T * 32 + (size_t)a.N * 68;
  size_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(m2rnn_bwd_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a0, const FwdArgs& replay, int dtype, hipStream_t stream) {
  BwdArgs a = a0;
  if (a.ckpt_every > kSub) {
    // states every kSub steps, replayed from the caller's checkpoints
    hipError_t e = launch_densify(replay, dtype, stream);
    if (e != hipSuccess) return e;
    a.H_ckpt = replay.H_ckpt;
    a.ckpt_every = kSub;
    a.nck = (a.T + kSub - 1) / kSub;
  }
  return dtype == 0 ? launch_bwd_t<float>(a, stream) : launch_bwd_t<bf16_t>(a, stream);
}

int backward_sub_steps() { return kSub; }

}  // namespace m2rnn

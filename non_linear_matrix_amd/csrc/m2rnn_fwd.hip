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
//  * a (b, n) head's 64 x 16 state sits in four MFMA accumulators (see
//    m2rnn_device.h), held by one, two or four waves for the whole sequence;
//  * H_{t-1} W is one v_mfma_f32_16x16x32_f16 per row tile: W^T in the A
//    operand (resident), hi/lo fp16 split of the fp32 state in the B operand
//    (fp32 inputs: four exact v_mfma_f32_16x16x4_f32);
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

// Launch shape: a workgroup serves HPW heads of one batch row; each head's four
// row tiles are spread over WPH = 4 / TPW waves (TPW tiles per wave).  More
// waves per head means more independent instruction streams per SIMD, which
// is what the per-step VALU work needs; the readout of a head then combines
// WPH per-wave partial sums through LDS.
template <int HPW, int TPW, int TC, bool DENSE = false>
struct FwdCfg {
  static constexpr int WPH = 4 / TPW;
  static constexpr int NWAVES = HPW * WPH;
  static constexpr int NT = 64 * NWAVES;
  // one staging buffer: K_s[TC][64], Q_s[TC][64] (not in the replay, which
  // has no readout), V_s[TC][HPW][16], F_s[TC][HPW][4]
  static constexpr int kQ = DENSE ? 0 : TC * 64;
  static constexpr int kBuf = TC * (64 + HPW * 20) + kQ;
  // per-wave readout partials and w_r (the replay has neither: its 37 KB let
  // four workgroups share a CU)
  static constexpr int kY = DENSE ? 0 : TC * HPW * WPH * 16;
  static constexpr int kWr = DENSE ? 0 : HPW * 16;
  static constexpr int kFloats = 2 * kBuf + kY + kWr;
  static constexpr int kBytes = kFloats * 4;
};

template <typename TIn, int HPW, int NT, int TC, bool GATE, bool WITH_Q = true>
struct FwdStager {
  typedef typename Vec4<TIn>::raw raw;
  static constexpr int NQK = (WITH_Q ? 2 : 1) * TC * 16;      // 4-vectors of k (and q)
  static constexpr int kQK = (NQK + NT - 1) / NT;
  static constexpr int kV = (TC * HPW * 4 + NT - 1) / NT;   // 4-vectors of v
  raw qk[kQK];
  raw vv[kV];
  TIn fr;   // f as stored, converted when staged

  // Every thread issues the same loads; a slot past the chunk's end, of a
  // missing head or beyond the staged counts reads valid data (step t0, head
  // n0) and is zeroed when staged.  No register of an in-flight load is then
  // merged or copied, and the conversions wait until the data is staged, so
  // the prefetch overlaps the chunk's steps.
  __device__ void load(const FwdArgs& a, int b, int n0, int t0, int t_end, int tid) {
#pragma unroll
    for (int r = 0; r < kQK; ++r) {
      const int u = tid + r * NT;           // [0, NQK)
      const int which = WITH_Q ? u / (TC * 16) : 1;   // 0: q, 1: k
      const int t = (u / 16) % TC, e0 = (u % 16) * 4;
      const bool ok = u < NQK && t0 + t < t_end;
      const TIn* src = (const TIn*)(which == 1 ? a.k : a.q);
      qk[r] = Vec4<TIn>::load(src + ((size_t)b * a.T + t0 + (ok ? t : 0)) * 64 + (ok ? e0 : 0));
    }
#pragma unroll
    for (int r = 0; r < kV; ++r) {
      const int u = tid + r * NT;           // [0, TC*HPW*4)
      const int t = u / (HPW * 4), h = (u / 4) % HPW, c4 = u % 4;
      const bool ok = u < TC * HPW * 4 && t0 + t < t_end && n0 + h < a.N;
      vv[r] = Vec4<TIn>::load((const TIn*)a.v + (((size_t)b * a.T + t0 + (ok ? t : 0)) * a.N + n0 + (ok ? h : 0)) * 16 +
                              (ok ? 4 * c4 : 0));
    }
    {
      const int t = tid / HPW, h = tid % HPW;
      const bool ok = tid < TC * HPW && t0 + t < t_end && n0 + h < a.N;
      const TIn* fsrc = (const TIn*)(GATE ? a.ga : a.f);   // f, or the gate's pre-activation
      fr = fsrc[((size_t)b * a.T + t0 + (ok ? t : 0)) * a.N + n0 + (ok ? h : 0)];
    }
  }

  // galpha, gbeta: the gate parameters of head n0 + tid % HPW (gate mode)
  __device__ void store(float* buf, const FwdArgs& a, int n0, int t0, int t_end, int tid, float galpha,
                        float gbeta) const {
    float* K_s = buf;
    float* Q_s = buf + TC * 64;   // with q only
    float* V_s = buf + (WITH_Q ? 2 : 1) * TC * 64;
    float* F_s = V_s + TC * HPW * 16;
#pragma unroll
    for (int r = 0; r < kQK; ++r) {
      int u = tid + r * NT;
      if (u < NQK) {
        int which = WITH_Q ? u / (TC * 16) : 1;
        int t = (u / 16) % TC, e0 = (u % 16) * 4;
        f4 x = Vec4<TIn>::to_f4(qk[r]);
        if (t0 + t >= t_end) x = f4{0.f, 0.f, 0.f, 0.f};
        // element e = 16 j + m goes to [t][m][j]: a lane with column m reads
        // its tiles' values as one contiguous word.
        float* dst = (which ? K_s : Q_s) + t * 64;
        float sc = which ? kScale : kInvScale;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int e = e0 + i;
          dst[(e % 16) * 4 + e / 16] = x[i] * sc;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kV; ++r) {
      int u = tid + r * NT;
      if (u < TC * HPW * 4) {
        const int t = u / (HPW * 4), h = (u / 4) % HPW;
        f4 x = Vec4<TIn>::to_f4(vv[r]);
        if (t0 + t >= t_end || n0 + h >= a.N) x = f4{0.f, 0.f, 0.f, 0.f};
        *(f4*)(V_s + u * 4) = x;
      }
    }
    if (tid < TC * HPW) {
      const int t = tid / HPW, h = tid % HPW;
      float ff = 1.0f;
      if (t0 + t < t_end && n0 + h < a.N) ff = GATE ? gate_value(to_f32(fr), galpha, gbeta).f : to_f32(fr);
      const float gg = 1.0f - ff;
      *(f4*)(F_s + tid * 4) = f4{ff, kScale * gg, -2.0f * kScale * gg, 0.0f};
    }
  }
};

// The TPW per-tile values a lane needs (k or q at rows 16 j + m of its tiles).
template <int TPW> struct TileVals { float v[TPW]; };
template <int TPW> __device__ __forceinline__ TileVals<TPW> load_tiles(const float* p) {
  TileVals<TPW> r;
  if constexpr (TPW == 4) {
    f4 x = *(const f4*)p;
    r.v[0] = x[0]; r.v[1] = x[1]; r.v[2] = x[2]; r.v[3] = x[3];
  } else if constexpr (TPW == 2) {
    f2 x = *(const f2*)p;
    r.v[0] = x[0]; r.v[1] = x[1];
  } else {
    r.v[0] = *p;
  }
  return r;
}

// DENSE = false: the forward scan proper (y, H_T, optional checkpoints).
// DENSE = true: the backward's replay.  Every workgroup takes one checkpoint
// chunk [c * src_every, (c+1) * src_every) of HPW heads, restarts from the
// stored H there and writes H every ckpt_every steps (no readout), so all
// chunks of a sequence run in parallel.
template <typename TIn, int HPW, int TPW, int TC, bool DENSE, bool GATE>
__global__ __launch_bounds__(256 * HPW / TPW) void m2rnn_fwd_kernel(FwdArgs a) {
  typedef FwdCfg<HPW, TPW, TC, DENSE> Cfg;
  constexpr int WPH = Cfg::WPH;
  extern __shared__ float smem[];
  float* ystage = smem + 2 * Cfg::kBuf;
  float* wr_s = ystage + Cfg::kY;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, g = lane / 16, m = lane % 16;
  const int hw = w / WPH, ts = w % WPH, j0 = ts * TPW;   // head in group, tile set, first tile
  const int ngroups = (a.N + HPW - 1) / HPW;
  int blk = blockIdx.x;
  if constexpr (DENSE) {
    static_assert(Cfg::NT == 256, "the gradient-scale role runs on 256 threads");
    if (blk < a.amax_wgs) {   // uniform over the workgroup
      grad_absmax_part(a.amax_dy, a.amax_ndy4, a.amax_dH, a.amax_ndh4, a.amax_part, blk, a.amax_wgs, smem);
      return;
    }
    blk -= a.amax_wgs;
  }
  const int n0 = (blk % ngroups) * HPW;
  blk /= ngroups;
  int tb = 0, te = a.T;
  if constexpr (DENSE) {
    const int chunk = blk % a.src_nck;
    blk /= a.src_nck;
    tb = chunk * a.src_every;
    te = min(a.T, tb + a.src_every);
  }
  const int b = blk;
  const int n = n0 + hw;
  const bool live = n < a.N;

  WOperand<TIn> Aw;
  Aw.load(live ? (const TIn*)a.W + (size_t)n * 256 : nullptr, g, m);
  if (!DENSE && tid < HPW * 16) {
    const int hh = tid / 16;
    wr_s[tid] = n0 + hh < a.N ? to_f32(((const TIn*)a.wr)[(size_t)(n0 + hh) * 16 + tid % 16]) : 0.0f;
  }

  f4 P[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) P[j] = f4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    // the restart state: a stored checkpoint (replay) or the caller's H_0
    const float* src = nullptr;
    if constexpr (DENSE) src = a.H_src + (((size_t)b * a.N + n) * a.src_nck + tb / a.src_every) * 1024;
    else if (a.H_0) src = a.H_0 + ((size_t)b * a.N + n) * 1024;
    if (src) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) P[j] = *(const f4*)(src + (16 * (j0 + j) + m) * 16 + 4 * g) * kScale;
    }
  }

  // gate parameters of the head whose f this thread stages
  float galpha = 0.0f, gbeta = 0.0f;
  if (GATE && tid < TC * HPW && n0 + tid % HPW < a.N) {
    galpha = to_f32(((const TIn*)a.galpha)[n0 + tid % HPW]);
    gbeta = to_f32(((const TIn*)a.gbeta)[n0 + tid % HPW]);
  }

  const int nchunks = (te - tb + TC - 1) / TC;
  {
    FwdStager<TIn, HPW, Cfg::NT, TC, GATE, !DENSE> st;
    st.load(a, b, n0, tb, te, tid);
    st.store(smem, a, n0, tb, te, tid, galpha, gbeta);
  }
  __syncthreads();

  // next step whose incoming state is checkpointed
  int ck_idx = a.H_ckpt ? (tb + a.ckpt_every - 1) / a.ckpt_every : 0;   // its checkpoint slot
  int next_ck = a.H_ckpt ? ck_idx * a.ckpt_every : a.T;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = tb + c * TC;
    const bool more = c + 1 < nchunks;
    // prefetch the next chunk (the last chunk fetches itself again and stages
    // it into the buffer no one reads).  Waves with steps to run issue it in
    // their first step: loads still in flight where the step loop (which
    // holds the checkpoint stores) is entered would be waited for there.
    const int tn = more ? t0 + TC : t0;
    // Wave priorities: the waves of a SIMD start the chunk together and
    // issue goes to the oldest ready wave, so the youngest would run its last
    // steps alone while the others wait at the barrier.  Each wave steps its
    // priority down (3, 2, 1, 0) over the four quarters of the chunk, which
    // gives the issue slots to the waves that are behind.
    __builtin_amdgcn_s_setprio(3);
    FwdStager<TIn, HPW, Cfg::NT, TC, GATE, !DENSE> st;
    if (DENSE || !live) st.load(a, b, n0, tn, te, tid);

    const float* buf = smem + (c & 1) * Cfg::kBuf;
    const float* K_s = buf;
    const float* Q_s = buf + TC * 64;   // not in the replay
    const float* V_s = buf + Cfg::kQ + TC * 64;
    const float* F_s = V_s + TC * HPW * 16;
    const int steps = min(TC, te - t0);
    if (live) {
      auto ckpt = [&](int t) {
        if (t == next_ck) {
          const size_t at = (((size_t)b * a.N + n) * a.nck + ck_idx) * 1024;
          next_ck += a.ckpt_every;
          ++ck_idx;
          if constexpr (DENSE && sizeof(TIn) == 2) {
            // the replay's states for the bf16-input sweep: c H in fp16 (the
            // sweep's contractions round the state to fp16 anyway)
#pragma unroll
            for (int j = 0; j < TPW; ++j)
              *(h4*)((_Float16*)a.H_ckpt + at + (16 * (j0 + j) + m) * 16 + 4 * g) = to_half4(P[j]);
          } else {
#pragma unroll
            for (int j = 0; j < TPW; ++j)   // the replay's states stay scaled by c (only the sweep reads them)
              *(f4*)(a.H_ckpt + at + (16 * (j0 + j) + m) * 16 + 4 * g) = DENSE ? P[j] : P[j] * kInvScale;
          }
        }
      };
      auto step_priority = [](int tt) {
        if (tt == TC / 4) __builtin_amdgcn_s_setprio(2);
        else if (tt == TC / 2) __builtin_amdgcn_s_setprio(1);
        else if (tt == 3 * TC / 4) __builtin_amdgcn_s_setprio(0);
      };
      auto step = [&](int tt) {
        const TileVals<TPW> kq = load_tiles<TPW>(K_s + tt * 64 + m * 4 + j0);   // c k[16j+m]
        TileVals<TPW> qq = {};                                                  // q[16j+m] / c
        if constexpr (!DENSE) qq = load_tiles<TPW>(Q_s + tt * 64 + m * 4 + j0);
        const f4 vv = *(const f4*)(V_s + (tt * HPW + hw) * 16 + 4 * g);
        const f4 fc = *(const f4*)(F_s + (tt * HPW + hw) * 4);                 // f, c(1-f), -2c(1-f)
        // The tiles' elements are independent once the contractions are
        // issued; the stages below are written element-wide so that the
        // transcendental latencies overlap.
        f4 x[TPW], hg[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) x[j] = Aw.times_state(P[j]);   // c (H W)^T tile
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[j][i] = fmaf(kq.v[j], vv[i], x[j][i]);                // c (H W + k v^T)
            hg[j][i] = fmaf(fc[0], P[j][i], fc[1]);                 // f P + c (1 - f)
          }
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[j][i] = __builtin_amdgcn_exp2f(x[j][i]) + 1.0f;
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[j][i] = __builtin_amdgcn_rcpf(x[j][i]);  // (1 - tanh) / 2
        f4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            P[j][i] = fmaf(fc[2], x[j][i], hg[j][i]);               // f P + c (1 - f) tanh
            p[i] = fmaf(P[j][i], qq.v[j], p[i]);
          }
        if constexpr (!DENSE) {
          // lane m ends with the sum for value channel 4 g + c(m); every lane
          // stores it (lanes m, m + 4, m + 8, m + 12 hold bitwise the same sum)
          const float ys = row_sum16x4(p, m);
          ystage[((tt * HPW + hw) * WPH + ts) * 16 + 4 * g + ((m & 1) << 1) + ((m >> 1) & 1)] = ys;
        }
      };
      // In the forward, a whole chunk whose checkpoints (if any) all fall on
      // every fourth step runs four steps per iteration: the checkpoint test
      // and the loop control once per four steps, the LDS offsets folded into
      // the reads.  (The replay, which stores every fourth state, measured
      // slightly slower this way and keeps the step loop.)
      if (!DENSE && steps == TC && (!a.H_ckpt || ((a.ckpt_every & 3) == 0 && ((next_ck - t0) & 3) == 0))) {
        for (int tt0 = 0; tt0 < TC; tt0 += 4) {
          if (!DENSE && tt0 == 0) st.load(a, b, n0, tn, te, tid);
          step_priority(tt0);
          ckpt(t0 + tt0);
#pragma unroll
          for (int u = 0; u < 4; ++u) step(tt0 + u);
        }
      } else {
        for (int tt = 0; tt < steps; ++tt) {
          if (!DENSE && tt == 0) st.load(a, b, n0, tn, te, tid);
          step_priority(tt);
          ckpt(t0 + tt);
          step(tt);
        }
      }
    }
    __syncthreads();
    // y = (sum of the per-wave partials) + w_r * v, rows [t][n0 .. n0+HPW)[16]
#pragma unroll
    for (int r = 0; r < (DENSE ? 0 : (TC * HPW * 4 + Cfg::NT - 1) / Cfg::NT); ++r) {
      const int u = tid + r * Cfg::NT;
      const int tt = u / (HPW * 4), hh = (u / 4) % HPW, c4 = u % 4;
      if (u < TC * HPW * 4 && tt < steps && n0 + hh < a.N) {
        f4 acc = *(const f4*)(ystage + ((tt * HPW + hh) * WPH) * 16 + 4 * c4);
#pragma unroll
        for (int ws = 1; ws < WPH; ++ws) acc += *(const f4*)(ystage + ((tt * HPW + hh) * WPH + ws) * 16 + 4 * c4);
        const f4 vres = *(const f4*)(V_s + (tt * HPW + hh) * 16 + 4 * c4);
        const f4 wres = *(const f4*)(wr_s + hh * 16 + 4 * c4);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wres[i], vres[i], acc[i]);
        *(f4*)(a.y + (((size_t)b * a.T + t0 + tt) * a.N + n0 + hh) * 16 + 4 * c4) = acc;
      }
    }
    st.store(smem + ((c + 1) & 1) * Cfg::kBuf, a, n0, tn, te, tid, galpha, gbeta);
    __syncthreads();
  }

  if (live && !DENSE) {
    float* dst = a.H_T + ((size_t)b * a.N + n) * 1024;
#pragma unroll
    for (int j = 0; j < TPW; ++j) *(f4*)(dst + (16 * (j0 + j) + m) * 16 + 4 * g) = P[j] * kInvScale;
  }
}

template <typename TIn, int HPW, int TPW, int TC, bool DENSE = false, bool GATE = false>
static hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  typedef FwdCfg<HPW, TPW, TC, DENSE> Cfg;
  static_assert(Cfg::kBytes <= 64 * 1024, "forward LDS budget");
  const int ngroups = (a.N + HPW - 1) / HPW;
  dim3 grid((unsigned)(a.B * ngroups * (DENSE ? a.src_nck : 1) + (DENSE ? a.amax_wgs : 0))), block(Cfg::NT);
  hipLaunchKernelGGL((m2rnn_fwd_kernel<TIn, HPW, TPW, TC, DENSE, GATE>), grid, block, Cfg::kBytes, stream, a);
  return hipGetLastError();
}

// Workgroup shape by the number of (batch row, head) chains.  Every head
// needs four tile-steps per time step, and the waves of a workgroup share one
// CU.  Many chains: four heads per workgroup, one head per wave, which issues
// the fewest instructions per head-step.  Few chains would then leave most
// CUs idle, so each head gets its own workgroup with one tile per wave (its
// four waves on the four SIMDs of a CU, the readout partials summed through
// LDS once per chunk); in between, two heads of two waves each.
constexpr long long kFewChains = 512, kMidChains = 1536;

template <typename TIn, bool GATE>
static hipError_t dispatch_fwd_shape(const FwdArgs& a, hipStream_t stream) {
  const long long chains = (long long)a.B * a.N;
  if (chains <= kFewChains) return launch_fwd<TIn, 1, 1, 32, false, GATE>(a, stream);
  if (chains <= kMidChains) return launch_fwd<TIn, 2, 2, 32, false, GATE>(a, stream);
  return launch_fwd<TIn, 4, 4, 32, false, GATE>(a, stream);
}

template <typename TIn>
static hipError_t dispatch_fwd(const FwdArgs& a, hipStream_t stream) {
  return a.ga ? dispatch_fwd_shape<TIn, true>(a, stream) : dispatch_fwd_shape<TIn, false>(a, stream);
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

__global__ void copy_kernel(float* dst, const float* src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) dst[i] = src[i];
}

hipError_t launch_copy(float* dst, const float* src, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, src, n);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? dispatch_fwd<float>(a, stream) : dispatch_fwd<bf16_t>(a, stream);
}

hipError_t launch_densify(const FwdArgs& a, int dtype, hipStream_t stream) {
  if (a.ga)
    return dtype == 0 ? launch_fwd<float, 4, 4, 32, true, true>(a, stream)
                      : launch_fwd<bf16_t, 4, 4, 32, true, true>(a, stream);
  return dtype == 0 ? launch_fwd<float, 4, 4, 32, true>(a, stream) : launch_fwd<bf16_t, 4, 4, 32, true>(a, stream);
}

}  // namespace m2rnn

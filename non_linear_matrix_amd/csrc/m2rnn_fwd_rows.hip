// m2rnn_fwd_rows.hip -- forward scan of the M2RNN recurrence for few
// (batch, head) chains, one state element per lane.
//
// Method: M2RNN paper-discussion slides (reading of arXiv:2603.14360v2),
// slide "Write, transform, retain, and read a matrix state" (paper
// Eqs. (10)-(12)):  Z_t = tanh(H_{t-1} W + k_t v_t^T),
// H_t = f_t H_{t-1} + (1 - f_t) Z_t,  y_t = H_t^T q_t + w_r (.) v_t, with q_t,
// k_t shared by the value heads (slide "Shared queries and keys buy more
// recurrent capacity", paper Alg. 1).  Time stays sequential per head (slide
// "Efficient tiles do not remove the sequential dependency").
//
// The MFMA forward (m2rnn_fwd.hip) holds a head's state in at most four
// waves, one per 16-row tile.  With few chains (B N <= kRowsMaxChains) that
// leaves most SIMDs idle and every time step costs the whole dependent chain
// of a tile step.  The rows of H never mix in the recurrence (only the
// readout sums over them), so here a head's 64 rows are spread over 16 waves
// in four workgroups, and each lane holds one state element:
//
//  * lane (r, j) of wave w in row group g holds P = c H[row][j], c = 2 / ln 2,
//    row = 16 g + 4 w + r;
//  * (H W)[row][j] = sum_i H[row][i] W[i][j] is 16 fp32 FMAs whose first
//    factor comes from lane i of the lane's own 16-lane row (DPP
//    row_newbcast), with W's column j resident in registers: exact fp32
//    products, in four interleaved partial sums;
//  * the rank-1 term, tanh as 1 - 2 / (1 + 2^{c x}) and the gate follow as in
//    the MFMA forward;
//  * each lane's readout product P q goes to LDS; once per chunk the
//    workgroup sums its 16 rows, and m2rnn_fwd_rows_reduce_kernel sums the
//    four row groups from per-group partial sums in the caller's workspace,
//    in a fixed order (deterministic), and adds w_r (.) v;
//  * q, k (this group's 16 rows), v and f stream through LDS in chunks of
//    kRowsTC steps, double-buffered and prefetched into registers one chunk
//    ahead.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

namespace {

constexpr int kRowsTC = 32;     // steps per staged chunk
constexpr int kRowsNT = 256;    // threads per workgroup: four waves, 16 rows

// sum over i = 0..15 of P(lane i of this lane's 16-lane row) * w[i], in four
// interleaved partial sums.  The DPP read of P needs two wait states after
// the VALU write of P, which the s_nop 1 at the head of the block provides
// (the compiler does not look inside the block); nothing inside the block
// writes P, and the early-clobber outputs keep the partial sums out of the
// inputs' registers.
__device__ __forceinline__ float row_contract(float P, const float (&w)[16]) {
  float a0, a1, a2, a3;
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %4, %5 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %4, %6 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %4, %7 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %4, %8 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %10 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %11 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %12 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %13 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %14 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %15 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %20 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
      : "v"(P), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "v"(w[8]),
        "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15]));
  return (a0 + a1) + (a2 + a3);
}

// Staging of one chunk (kRowsTC steps from t0; steps at or past t_end are
// staged as f = 1 with q = k = v = 0, an exact identity on the state) into an
// LDS buffer: kq [t][16 rows][c k, q / c], v [t][16], fc [t] = f, c (1 - f),
// -2 c (1 - f).  Every thread issues its loads unconditionally (addresses of
// missing steps and idle slots are clamped to valid data), so the prefetch
// registers are never merged or copied while their loads are in flight.
template <typename TIn, bool GATE>
struct RowsStager {
  static constexpr int EPC = 16 / (int)sizeof(TIn);   // elements per 16-byte chunk
  static constexpr int CPS = 16 / EPC;                // chunks per step per tensor
  static constexpr int NC = 3 * kRowsTC * CPS;        // q, k, v chunks
  static constexpr int R = (NC + kRowsNT - 1) / kRowsNT;
  u32x4 r[R];
  TIn fr;

  __device__ void load(const FwdArgs& a, int b, int n, int g, int t0, int t_end, int tid) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int u = tid + i * kRowsNT;
      const int kind = u / (kRowsTC * CPS), rem = u % (kRowsTC * CPS), t = rem / CPS, c = rem % CPS;
      const bool ok = u < NC && t0 + t < t_end;
      const size_t row = (size_t)b * a.T + t0 + (ok ? t : 0);
      const TIn* p;
      if (kind == 1) p = (const TIn*)a.k + row * 64 + 16 * g + c * EPC;
      else if (kind == 2) p = (const TIn*)a.v + (row * a.N + n) * 16 + c * EPC;
      else p = (const TIn*)a.q + row * 64 + 16 * g + (kind == 0 ? c * EPC : 0);
      r[i] = *(const u32x4*)p;
    }
    const bool fok = tid < kRowsTC && t0 + tid < t_end;
    const TIn* fsrc = (const TIn*)(GATE ? a.ga : a.f);
    fr = fsrc[((size_t)b * a.T + t0 + (fok ? tid : 0)) * a.N + n];
  }

  __device__ void store(float* kq, float* vs, f4* fs, int t0, int t_end, int tid, float galpha, float gbeta) const {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int u = tid + i * kRowsNT;
      if (u < NC) {
        const int kind = u / (kRowsTC * CPS), rem = u % (kRowsTC * CPS), t = rem / CPS, c = rem % CPS;
        float x[EPC];
        if constexpr (sizeof(TIn) == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(r[i][e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(r[i][e] << 16);
            x[2 * e + 1] = __uint_as_float(r[i][e] & 0xffff0000u);
          }
        }
        const bool ok = t0 + t < t_end;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float xv = ok ? x[e] : 0.0f;
          const int col = c * EPC + e;
          if (kind == 0) kq[(t * 16 + col) * 2 + 1] = xv * kInvScale;   // q / c
          else if (kind == 1) kq[(t * 16 + col) * 2] = xv * kScale;     // c k
          else vs[t * 16 + col] = xv;
        }
      }
    }
    if (tid < kRowsTC) {
      float ff = 1.0f;
      if (t0 + tid < t_end) ff = GATE ? gate_value(to_f32(fr), galpha, gbeta).f : to_f32(fr);
      const float gg = 1.0f - ff;
      fs[tid] = f4{ff, kScale * gg, -2.0f * kScale * gg, 0.0f};
    }
  }
};

template <typename TIn, bool GATE>
__global__ __launch_bounds__(kRowsNT) void m2rnn_fwd_rows_kernel(FwdArgs a) {
  __shared__ __align__(16) float kq_s[2][kRowsTC * 32];
  __shared__ __align__(16) float v_s[2][kRowsTC * 16];
  __shared__ f4 f_s[2][kRowsTC];
  // readout products P q of every lane, [t][column][row within the group],
  // 20 floats per (t, column) (16-byte aligned rows; two lanes per bank on write)
  __shared__ __align__(16) float ys[kRowsTC * 16 * 20];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, r = lane / 16, j = lane % 16;
  const int g = blockIdx.x % 4;
  const int n = (blockIdx.x / 4) % a.N;
  const int b = blockIdx.x / 4 / a.N;
  const int rw = 4 * w + r;            // row within the group
  const int row = 16 * g + rw;         // row of H
  const size_t head = (size_t)b * a.N + n;

  float wc[16];                        // column j of W
  {
    const TIn* Wn = (const TIn*)a.W + (size_t)n * 256;
#pragma unroll
    for (int i = 0; i < 16; ++i) wc[i] = to_f32(Wn[i * 16 + j]);
  }
  float P = a.H_0 ? a.H_0[head * 1024 + row * 16 + j] * kScale : 0.0f;
  float galpha = 0.0f, gbeta = 0.0f;
  if (GATE) {
    galpha = to_f32(((const TIn*)a.galpha)[n]);
    gbeta = to_f32(((const TIn*)a.gbeta)[n]);
  }

  const int nchunks = (a.T + kRowsTC - 1) / kRowsTC;
  {
    RowsStager<TIn, GATE> st;
    st.load(a, b, n, g, 0, a.T, tid);
    st.store(kq_s[0], v_s[0], f_s[0], 0, a.T, tid, galpha, gbeta);
  }
  __syncthreads();

  int ck_idx = 0;
  int next_ck = a.H_ckpt ? 0 : a.T;
  float* ypart = a.ypart + (head * 4 + g) * (size_t)a.T * 16;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kRowsTC;
    const int steps = min(kRowsTC, a.T - t0);
    const int tn = c + 1 < nchunks ? t0 + kRowsTC : t0;   // the last chunk stages itself again, unread
    RowsStager<TIn, GATE> st;
    st.load(a, b, n, g, tn, a.T, tid);
    const float* kq = kq_s[c & 1];
    const float* vs = v_s[c & 1];
    const f4* fs = f_s[c & 1];
    auto step = [&](int tt) {
      const f2 kqv = *(const f2*)(kq + (tt * 16 + rw) * 2);   // c k[row], q[row] / c
      const float vj = vs[tt * 16 + j];
      const f4 fc = fs[tt];
      float x = row_contract(P, wc);                           // c (H W)[row][j]
      x = fmaf(kqv[0], vj, x);                                 // + c k v^T
      const float hg = fmaf(fc[0], P, fc[1]);                  // f P + c (1 - f)
      const float rr = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x) + 1.0f);   // (1 - tanh) / 2
      P = fmaf(fc[2], rr, hg);                                 // f P + c (1 - f) tanh
      ys[(tt * 16 + j) * 20 + rw] = P * kqv[1];
    };
    if (steps == kRowsTC && (!a.H_ckpt || ((a.ckpt_every & 3) == 0 && ((next_ck - t0) & 3) == 0))) {
      for (int tt0 = 0; tt0 < kRowsTC; tt0 += 4) {
        if (t0 + tt0 == next_ck) {
          a.H_ckpt[(head * a.nck + ck_idx) * 1024 + row * 16 + j] = P * kInvScale;
          next_ck += a.ckpt_every;
          ++ck_idx;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) step(tt0 + u);
      }
    } else {
      for (int tt = 0; tt < steps; ++tt) {
        if (t0 + tt == next_ck) {
          a.H_ckpt[(head * a.nck + ck_idx) * 1024 + row * 16 + j] = P * kInvScale;
          next_ck += a.ckpt_every;
          ++ck_idx;
        }
        step(tt);
      }
    }
    __syncthreads();
    // this group's readout partials: the sum over its 16 rows, in a fixed order
    for (int u = tid; u < steps * 16; u += kRowsNT) {
      const f4* s = (const f4*)(ys + u * 20);   // u = tt * 16 + column
      const f4 x = (s[0] + s[1]) + (s[2] + s[3]);
      ypart[(size_t)t0 * 16 + u] = (x[0] + x[1]) + (x[2] + x[3]);
    }
    st.store(kq_s[(c + 1) & 1], v_s[(c + 1) & 1], f_s[(c + 1) & 1], tn, a.T, tid, galpha, gbeta);
    __syncthreads();
  }
  a.H_T[head * 1024 + row * 16 + j] = P * kInvScale;
}

// y[b][t][n][:] = ((part_0 + part_1) + (part_2 + part_3)) + w_r (.) v over the
// four row groups' partial readouts [b][n][g][t][16].
template <typename TIn>
__global__ __launch_bounds__(256) void m2rnn_fwd_rows_reduce_kernel(FwdArgs a) {
  const size_t total = (size_t)a.B * a.N * a.T * 4;
  const size_t gstride = (size_t)a.T * 16;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const int c4 = (int)(u % 4);
    size_t rest = u / 4;
    const size_t t = rest % a.T;
    rest /= a.T;
    const int n = (int)(rest % a.N);
    const size_t b = rest / a.N;
    const float* src = a.ypart + ((b * a.N + n) * 4) * gstride + t * 16 + 4 * c4;
    f4 acc = (*(const f4*)src + *(const f4*)(src + gstride)) +
             (*(const f4*)(src + 2 * gstride) + *(const f4*)(src + 3 * gstride));
    const size_t yo = ((b * a.T + t) * a.N + n) * 16 + 4 * c4;
    const f4 vres = Vec4<TIn>::to_f4(Vec4<TIn>::load((const TIn*)a.v + yo));
    const TIn* wr = (const TIn*)a.wr + (size_t)n * 16 + 4 * c4;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(to_f32(wr[i]), vres[i], acc[i]);
    *(f4*)(a.y + yo) = acc;
  }
}

template <typename TIn, bool GATE>
hipError_t launch_rows_t(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((m2rnn_fwd_rows_kernel<TIn, GATE>), dim3((unsigned)(a.B * a.N * 4)), dim3(kRowsNT), 0, stream,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t blocks = ((size_t)a.B * a.N * a.T * 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((m2rnn_fwd_rows_reduce_kernel<TIn>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

size_t forward_workspace_floats(int B, int T, int N) {
  if ((long long)B * N > kRowsMaxChains) return 0;
  return (size_t)B * N * 4 * T * 16;
}

hipError_t launch_forward_rows(const FwdArgs& a, int dtype, hipStream_t stream) {
  if (a.ga) return dtype == 0 ? launch_rows_t<float, true>(a, stream) : launch_rows_t<bf16_t, true>(a, stream);
  return dtype == 0 ? launch_rows_t<float, false>(a, stream) : launch_rows_t<bf16_t, false>(a, stream);
}

}  // namespace m2rnn

// m2rnn_decode.hip -- one token of the M2RNN recurrence for every (b, n)
// head, the state held by the caller (decoding).
//
// Method: M2RNN paper-discussion slides (reading of arXiv:2603.14360v2),
// slide "Write, transform, retain, and read a matrix state" (paper Eqs.
// (10)-(12)) for a single step from the caller's H:
//     Z = tanh(H W + k v^T),  H' = f H + (1 - f) Z,  y = H'^T q + w_r (.) v,
// with q, k shared by the N heads of a batch row (slide "Shared queries and
// keys buy more recurrent capacity", paper Alg. 1).
//
// A step reads and writes 8 KB of state per head and computes little, so the
// kernel is one wave per head with nothing staged: the wave loads its head's
// state tiles, W and the token's q, k, v, f straight into registers, runs the
// step with the forward scan's arithmetic at four tiles per wave (the same
// operations in the same order, so the result is bit-identical to that
// forward's first step), reduces the readout within its 16-lane rows and
// writes y and the new state back in place.  Four heads share a workgroup;
// no barrier, no LDS.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

constexpr int kDecodeHeads = 4;   // waves (heads) per workgroup

template <typename TIn>
__global__ __launch_bounds__(64 * kDecodeHeads) void m2rnn_decode_kernel(DecodeArgs a) {
  const int lane = threadIdx.x % 64, g = lane / 16, m = lane % 16;
  const long long head = (long long)blockIdx.x * kDecodeHeads + threadIdx.x / 64;   // b N + n
  if (head >= (long long)a.B * a.N) return;   // the whole wave
  const int b = (int)(head / a.N), n = (int)(head % a.N);

  WOperand<TIn> Aw;
  Aw.load((const TIn*)a.W + (size_t)n * 256, g, m);
  // lane (g, m), tile j: state row 16 j + m, value columns 4 g .. 4 g + 3,
  // scaled by c = 2 / ln 2 (the forward's frame)
  float* H = a.H + (size_t)head * 1024;
  f4 P[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) P[j] = *(const f4*)(H + (16 * j + m) * 16 + 4 * g) * kScale;
  const TIn* qb = (const TIn*)a.q + (size_t)b * 64;
  const TIn* kb = (const TIn*)a.k + (size_t)b * 64;
  float kq[4], qq[4];   // c k and q / c of the lane's four rows
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kq[j] = to_f32(kb[16 * j + m]) * kScale;
    qq[j] = to_f32(qb[16 * j + m]) * kInvScale;
  }
  const TIn* vh = (const TIn*)a.v + (size_t)head * 16;
  const f4 vv = Vec4<TIn>::to_f4(Vec4<TIn>::load(vh + 4 * g));
  const float ff = to_f32(((const TIn*)a.f)[head]);
  const float gg = 1.0f - ff;
  const f4 fc = f4{ff, kScale * gg, -2.0f * kScale * gg, 0.0f};   // f, c(1-f), -2c(1-f)

  f4 x[4], hg[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = Aw.times_state(P[j]);   // c (H W)^T tile
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[j][i] = fmaf(kq[j], vv[i], x[j][i]);                  // c (H W + k v^T)
      hg[j][i] = fmaf(fc[0], P[j][i], fc[1]);                 // f P + c (1 - f)
    }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[j][i] = __builtin_amdgcn_exp2f(x[j][i]) + 1.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[j][i] = __builtin_amdgcn_rcpf(x[j][i]);   // (1 - tanh) / 2
  f4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      P[j][i] = fmaf(fc[2], x[j][i], hg[j][i]);               // f P + c (1 - f) tanh
      p[i] = fmaf(P[j][i], qq[j], p[i]);
    }
  // lane m ends with the sum over the 64 rows for value channel
  // e = 4 g + 2 (m & 1) + ((m >> 1) & 1); lanes m < 4 of each row write it
  const float ys = row_sum16x4(p, m);
  if (m < 4) {
    const int e = 4 * g + ((m & 1) << 1) + ((m >> 1) & 1);
    a.y[head * 16 + e] = fmaf(to_f32(((const TIn*)a.wr)[(size_t)n * 16 + e]), to_f32(vh[e]), ys);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) *(f4*)(H + (16 * j + m) * 16 + 4 * g) = P[j] * kInvScale;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
  const long long heads = (long long)a.B * a.N;
  if (heads == 0) return hipSuccess;
  const dim3 grid((unsigned)((heads + kDecodeHeads - 1) / kDecodeHeads)), block(64 * kDecodeHeads);
  if (dtype == 0)
    hipLaunchKernelGGL(m2rnn_decode_kernel<float>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(m2rnn_decode_kernel<bf16_t>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace m2rnn

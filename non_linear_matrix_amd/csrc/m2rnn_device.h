// m2rnn_device.h -- gfx950 device helpers shared by the M2RNN scan kernels.
//
// State layout ("transposed frame").  A head's K x V = 64 x 16 state H is held
// as four 16 x 16 row tiles j = 0..3 (rows kk = 16 j .. 16 j + 15).  Each tile
// lives in one MFMA 16x16 accumulator (4 VGPRs per lane) holding the
// TRANSPOSED tile: lane l = 16 g + m, register i holds
//      P[j][i] = c * H[kk = 16 j + m][v = 4 g + i],        c = 2 / ln 2,
// i.e. row (4g+i), column m of the 16x16 matrix H_tile^T.  In that layout the
// step's contraction (H W)^T = W^T H^T is an MFMA whose B operand is the
// accumulator itself, so the state never leaves registers between steps.
// The scale c turns tanh(x) = 1 - 2 / (1 + e^{2x}) into one v_exp_f32 of the
// scaled pre-activation (exp2(c x) = e^{2x}).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2rnn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kScale = 2.8853900817779268f;     // 2 / ln 2
constexpr float kInvScale = 0.34657359027997264f; // ln 2 / 2
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16_t {
  uint16_t bits;
};

// ---------------------------------------------------------------- input loads
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  typedef f4 raw;
  __device__ static raw load(const float* p) { return *(const f4*)p; }
  __device__ static f4 to_f4(raw r) { return r; }
  __device__ static raw zero() { return f4{0.f, 0.f, 0.f, 0.f}; }
};
template <> struct Vec4<bf16_t> {
  typedef uint2 raw;
  __device__ static raw load(const bf16_t* p) { return *(const uint2*)p; }
  __device__ static f4 to_f4(raw r) {
    return f4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
              __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
  }
  __device__ static raw zero() { return uint2{0u, 0u}; }
};

// ------------------------------------------------------------ forget gate
// f = exp(-alpha softplus(a + beta)) (slide "The gate preserves a direct path
// through time", paper Eqs. (13), (17)), with softplus(x) = max(x, 0) +
// log(1 + e^{-|x|}) so that no exponential overflows.  Also returns
// softplus(x) and sigmoid(x) = softplus'(x) for the backward.
// A wave-uniform pointer read back into scalar registers: the compiler then
// does not fold a per-lane offset into it and keep that sum in vector
// registers across a loop.
template <typename T>
__device__ __forceinline__ T* sgpr_ptr(T* p) {
  const unsigned long long u = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return (T*)(((unsigned long long)hi << 32) | lo);
}

struct GateVal { float f, sp, sig; };
__device__ __forceinline__ GateVal gate_value(float a, float alpha, float beta) {
  const float x = a + beta;
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);            // e^{-|x|}
  const float sp = fmaxf(x, 0.0f) + kLn2 * __builtin_amdgcn_logf(1.0f + e);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  GateVal g;
  g.sp = sp;
  g.sig = x >= 0.0f ? r : e * r;
  g.f = __builtin_amdgcn_exp2f(-alpha * sp * kLog2e);
  return g;
}

// ------------------------------------------------------- fp16 hi/lo splitting
// x = hi + lo with hi = fp16(x) and lo = fp16(x - hi), both round-to-nearest-
// even (v_cvt_pk_f16_f32).  x - hi is exact in fp32 and comes from one
// v_fma_mix_f32 that reads hi as the fp16 half of the packed register it
// already sits in.  For |x| <= c (every state element) the pair carries x to
// within 2^-22 |x| + 2^-25 (fp16 subnormals are kept), which is finer than a
// bf16 pair (2^-17 |x|) at the same cost in MFMA work and 4 fewer VALU
// instructions per four elements.
__device__ __forceinline__ float minus_half_lo(uint32_t hpk, float x) {   // x - (float)(low fp16 of hpk)
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hpk), "v"(x));
  return r;
}
__device__ __forceinline__ float minus_half_hi(uint32_t hpk, float x) {   // x - (float)(high fp16 of hpk)
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hpk), "v"(x));
  return r;
}
__device__ __forceinline__ void split2h(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{x0, x1}), h2));
  const float l0 = minus_half_lo(hi, x0), l1 = minus_half_hi(hi, x1);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{l0, l1}), h2));
}

// B operand of v_mfma_f32_16x16x32_f16 from an accumulator tile: k-slots
// 0..3 of lane group g carry hi(x[0..3]), slots 4..7 carry lo(x[0..3]).
__device__ __forceinline__ h8 split_operand(f4 x) {
  uint32_t h01, l01, h23, l23;
  split2h(x[0], x[1], h01, l01);
  split2h(x[2], x[3], h23, l23);
  return __builtin_bit_cast(h8, (u32x4{h01, h23, l01, l23}));
}

// ------------------------------------------- the per-step contraction W^T P
// Given a state tile in accumulator layout (lane 16g+m, register i holds
// P^T[4g+i][m]), returns the accumulator-layout tile (W^T P^T)[v'][m] =
// sum_v W[v][v'] P^T[v][m], i.e. the transposed tile of P W.
template <typename TIn> struct WOperand;

// bfloat16 inputs: W is exact in fp16 (for 2^-14 <= |W| <= 65504; smaller
// values round to within 2^-25); the fp32 state is split hi + lo and both
// halves ride in one v_mfma_f32_16x16x32_f16 (A = [W^T | W^T]).
template <> struct WOperand<bf16_t> {
  h8 a;
  __device__ void load(const bf16_t* Wn, int g, int m) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const _Float16 x = (_Float16)(Wn ? to_f32(Wn[(4 * g + s) * 16 + m]) : 0.0f);
      a[s] = a[s + 4] = x;
    }
  }
  __device__ f4 times_state(f4 p) const {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, split_operand(p), f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};

// float32 inputs: four exact v_mfma_f32_16x16x4_f32; accumulator register r
// is the B operand of instruction r as is.
template <> struct WOperand<float> {
  float a[4];
  __device__ void load(const float* Wn, int g, int m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = Wn ? Wn[(4 * g + r) * 16 + m] : 0.0f;
  }
  __device__ f4 times_state(f4 p) const {
    f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], p[r], d, 0, 0, 0);
    return d;
  }
};

// ------------------------- one fp16 pass, for the sweep's short replays only
// The backward's reverse sweep replays a few steps at a time from states the
// chunk replay computed at full precision (stored once rounded to fp16), so
// the rounding of a single fp16 pass acts over those few steps only and
// stays well inside the backward's bf16-input bar.  (Over a
// whole 64-step checkpoint chunk it does not: with a gate close to 1 the
// rounding errors of the state accumulate across the chunk, so the chunk
// replay keeps the split.)  Both factors are rounded once to fp16
// (v_cvt_pk_f16_f32: round to nearest even, subnormals kept; 11 significant
// bits, 8 times finer than bf16): P = c H is bounded by c, and a bf16 W is
// exact in fp16 for 2^-14 <= |W| <= 65504.  One v_mfma_f32_16x16x16_f16 per
// tile instead of the split.
__device__ __forceinline__ h4 to_half4(f4 x) {
  const h2 a = __builtin_convertvector((f2{x[0], x[1]}), h2);
  const h2 b = __builtin_convertvector((f2{x[2], x[3]}), h2);
  return h4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ f4 mfma_f16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// The step's contraction in one fp16 pass: A = W^T (lane 16g+m holds
// W[4g+s][m], s = 0..3), B = the accumulator tile as is.
struct WOperandF16 {
  h4 a;
  __device__ void load(const bf16_t* Wn, int g, int m) {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = (_Float16)(Wn ? to_f32(Wn[(4 * g + s) * 16 + m]) : 0.0f);
  }
  __device__ f4 times_state(f4 p) const { return times_half(to_half4(p)); }
  // the same from a tile already rounded to fp16
  __device__ f4 times_half(h4 ph) const { return mfma_f16(a, ph, f4{0.f, 0.f, 0.f, 0.f}); }
};

// The operand of the sweep's replay: one fp16 pass for bf16 inputs, the exact
// fp32 MFMAs for fp32 inputs (whose bar is 50 times tighter).
template <typename TIn> struct ReplayOperand { typedef WOperand<TIn> type; };
template <> struct ReplayOperand<bf16_t> { typedef WOperandF16 type; };

// ------------------------------------------------- the gradients' scale
// Largest finite magnitude of dy and dH_T, the gradients that enter the
// backward's sweep, as kAmaxParts per-workgroup partial maxima; every sweep
// workgroup reduces them to the same scale.  NaN and infinite values are
// skipped, so a non-finite gradient of one chain leaves the scale, and with
// it every other chain's results, as they would be without it.  Run by
// workgroups of 256 threads: those of their own launch, or extra workgroups
// of the chunk replay, which then overlap the replay's arithmetic.
constexpr int kAmaxParts = 128;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float finite_abs(float x) {
  const float a = fabsf(x);
  return a <= 3.4028235e38f ? a : 0.0f;
}
__device__ __forceinline__ float absmax4(f4 v) {
  return fmaxf(fmaxf(finite_abs(v[0]), finite_abs(v[1])), fmaxf(finite_abs(v[2]), finite_abs(v[3])));
}
// Workgroup wg of nwg: the maximum over its contiguous slice of dy (eight
// 4 KB loads in flight at a time) and its share of dH_T, into part[wg].
// wm: four floats of LDS.
__device__ __forceinline__ void grad_absmax_part(const float* dy, size_t ndy4, const float* dH, size_t ndh4,
                                                 float* part, int wg, int nwg, float* wm) {
  const size_t per = (ndy4 + nwg - 1) / nwg;
  const size_t lo = min(ndy4, (size_t)wg * per), hi = min(ndy4, lo + per);
  const f4* p = (const f4*)dy;
  float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    f4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * 256];
    m0 = fmaxf(m0, fmaxf(absmax4(v[0]), absmax4(v[1])));
    m1 = fmaxf(m1, fmaxf(absmax4(v[2]), absmax4(v[3])));
    m2 = fmaxf(m2, fmaxf(absmax4(v[4]), absmax4(v[5])));
    m3 = fmaxf(m3, fmaxf(absmax4(v[6]), absmax4(v[7])));
  }
  for (; i < hi; i += 256) m0 = fmaxf(m0, absmax4(p[i]));
  if (dH) {
    const f4* h = (const f4*)dH;
    for (size_t k = (size_t)wg * 256 + threadIdx.x; k < ndh4; k += (size_t)nwg * 256) m1 = fmaxf(m1, absmax4(h[k]));
  }
  const float mx = wave_max(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
  if (threadIdx.x % 64 == 0) wm[threadIdx.x / 64] = mx;
  __syncthreads();
  if (threadIdx.x == 0) part[wg] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

// ------------------------------------------------------ cross-lane reductions
// (every control used here reads a lane of the same row, so bound_ctrl never
// applies; setting it lets the compiler fold the move into the add)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// Sum over the 16 lanes of each row (lanes 16g .. 16g+15); every lane of the
// row ends with the row sum.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  x += dpp<0x141>(x); // row_half_mirror
  x += dpp<0x128>(x); // row_ror:8 (lane m adds lane m +- 8)
  return x;
}
// Row sums of four values per lane at once (each 16-lane row reduces its own
// x[0..3]).  Returns, in lane m of the row, the row sum of x[c] with
// c = 2 (m & 1) + ((m >> 1) & 1): two halving exchanges (each lane keeps half
// of its values and adds the partner's matching half: lanes m ^ 1, then
// m ^ 2), then two rotations within the row add the four quads: by 8 first,
// which leaves lanes m and m + 8 with the same pair sum, then by 4, so that
// lanes m, m + 4, m + 8 and m + 12 add the same two values (in either order:
// IEEE addition commutes) and end with bitwise the same sum.
__device__ __forceinline__ float row_sum16x4(f4 x, int m) {
  const bool b0 = (m & 1) != 0, b1 = (m & 2) != 0;
  const float k0 = b0 ? x[2] : x[0], k1 = b0 ? x[3] : x[1];
  const float s0 = b0 ? x[0] : x[2], s1 = b0 ? x[1] : x[3];
  const float y0 = k0 + dpp<0xB1>(s0), y1 = k1 + dpp<0xB1>(s1);   // quad_perm [1,0,3,2]
  float z = (b1 ? y1 : y0) + dpp<0x4E>(b1 ? y0 : y1);              // quad_perm [2,3,0,1]
  z += dpp<0x128>(z);                                               // row_ror:8
  z += dpp<0x124>(z);                                               // row_ror:4
  return z;
}

}  // namespace m2rnn

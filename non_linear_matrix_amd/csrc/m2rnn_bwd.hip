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
//  * the states the sweep restarts from: when the caller's checkpoints are
//    sparser than kSub steps, a replay launch (the forward kernel in DENSE
//    mode, m2rnn_fwd.hip) restarts every checkpoint chunk in parallel and
//    writes c H every kSub steps into the workspace (for bf16 inputs rounded
//    once to fp16, the precision the sweep's contractions take the state in:
//    half the bytes of the largest write and read of the backward);
//  * one wave64 owns one 16-row tile of one (b, n) head (rows of H never mix
//    in the recurrence; only the reductions couple them), so a head is four
//    waves of one workgroup and a workgroup holds HPW heads of a batch row;
//    per kSub-step sub-chunk, latest first, the wave replays the steps keeping
//    H_{t-1} and Z_t in registers, then walks them back;
//  * C_{t-1}^T = f R^T + W D^T is one v_mfma_f32_16x16x16_f16 per step (W in
//    the A operand, D^T rounded once to fp16 in B, f R^T as the accumulator
//    input; four exact fp32 MFMAs for fp32 inputs), in the same transposed
//    frame as the forward, so C stays in registers.  For the fp16 rounding,
//    dy and dH_T enter scaled by a power of two that puts their largest
//    magnitude in [1/4, 1/2) (every gradient is linear in them; the outputs
//    are scaled back exactly), so D sits well inside fp16's range whatever
//    the scale of the caller's gradients;
//  * the sweep's few-step replays run one fp16 pass per step
//    (m2rnn_device.h) from states that the chunk replay computed at the
//    forward's precision;
//  * dW needs a contraction over the rows, which live on lanes: each step the
//    wave writes its H_{t-1} and D tiles to LDS and reads them back in MFMA
//    operand layout one step later (one bf16 MFMA on rounded factors for
//    bf16 inputs, four exact fp32 MFMAs for fp32 inputs), accumulated in
//    registers over the whole sequence;
//  * per-lane partials of df, dv, dq and dk go to LDS and are reduced once per
//    sub-chunk; the sums over workgroups (dq, dk) and batch rows (dW, dw_r)
//    are a second, fixed-order reduction kernel.
#include <mutex>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

constexpr int kSub = 4;  // steps between restart states; their H_{t-1}, Z_t stay in registers

// The power of two sig = 2^-e that puts mx sig in [1/4, 1/2), and 1 / sig;
// 1 when mx is zero or not finite.
__device__ __forceinline__ void grad_scale(float mx, float& sig, float& isig) {
  sig = isig = 1.0f;
  if (mx > 0.0f && mx <= 3.4028235e38f) {
    int e;
    frexpf(mx, &e);                          // mx in [2^(e-1), 2^e)
    e = min(max(e + 1, -120), 120);
    sig = ldexpf(1.0f, -e);
    isig = ldexpf(1.0f, e);
  }
}

// The df role's layout: pair p = s HPW + h of a sub-chunk goes to df wave
// p / 4 as its value o = p % 4, which sum4_over_lanes leaves in lane row
// r = 2 (o & 1) + (o >> 1) (the map is its own inverse).  gate_slot is the
// (wave, row) slot of (step s, head h).
template <int HPW>
__device__ __forceinline__ int gate_slot(int s, int h) {
  const int p = s * HPW + h, o = p & 3;
  return (p >> 2) * 4 + 2 * (o & 1) + (o >> 1);
}

template <int HPW, bool GATE, bool HALF>
struct BwdCfg {
  // the reduction pass gives each wave a fixed role (lane = (step, 16 values))
  static_assert((HPW == 1 || HPW == 2 || HPW == 4) && kSub == 4, "backward workgroup shape");
  // pass roles: dq, dk; one dv wave per head; df waves, wave d for the four
  // (step, head) pairs p = 4 d .. 4 d + 3 of the sub-chunk, p = step HPW + head
  static constexpr int kDvWave = 2, kDfWave = 2 + HPW, kRoleWaves = 2 + HPW + HPW;
  static constexpr int NWAVES = HPW * 4;
  static constexpr int NT = 64 * NWAVES;
  // per staged step: K_s[64] (c k), Q_s[64] (q), V_s[HPW][16], F_s[HPW][4],
  // U_s[HPW][16], Kp_s[64] (k permuted, [tile][g][r] = row 16 tile + 4 r + g:
  // c k in fp32 for fp32 inputs, k in fp16 for bf16 inputs),
  // with the gate G_s[HPW][2] (df -> da and df -> dalpha factors, in the df
  // waves' row order, slot gate_slot(s, h)), and for bf16 inputs UV_s
  // [HPW][2][4][8] fp16, the A operand of the joint dq, dk contraction (u in
  // the first, v in the second half of the 16 rows)
  static constexpr int kStep = 192 + HPW * (36 + (GATE ? 2 : 0) + (HALF ? 32 : 0));
  static constexpr int kBuf = kSub * kStep;
  // Buffering.  bf16 inputs (HALF): three staging buffers and two sets of
  // partials, so that one barrier per sub-chunk suffices: the sweep of
  // sub-chunk i writes partials set i % 2 while waves still in the pass of
  // i - 1 read the other set, and the pass of i stages sub-chunk i + 2 while
  // the buffer of i + 1 is complete.  fp32 inputs, whose transposes and
  // partials take four times the LDS, keep two staging buffers and one set,
  // with a second barrier after the pass.
  static constexpr int kNStage = HALF ? 3 : 2;
  static constexpr int kNPart = HALF ? 2 : 1;
  // per wave, two slots of {H_{t-1} tile, D tile}.  fp32: a tile is stored as
  // [v / 4][kk][v % 4] with a 72-float stride between the v / 4 blocks, which
  // keeps both the 16-byte writes and the operand-layout reads free of bank
  // conflicts (LDS: 32 four-byte banks, a 4-byte access served per 32 lanes,
  // a 16-byte access per 8 lanes); bf16: 64 chunks of four fp16 per tile (the
  // layout is described at the sweep)
  static constexpr int kXs = 72;
  static constexpr int kTile = 3 * kXs + 64;
  static constexpr int kXw = HALF ? 2 * 2 * 64 * 2 : 4 * kTile;   // floats per wave
  static constexpr int kXpose = NWAVES * kXw;
  // per-lane partials of one sub-chunk:
  //   qk: [s][dq | dk][h] x kQKRow.  fp32 inputs: 256 per block, [g][64
  //       rows], partials over the four values of lane group g, the 4-row
  //       quads of group g rotated by 4 g quads (conflict-free writes,
  //       16-byte reads); bf16 inputs: 64 per block, the whole sum of each
  //       row (the joint MFMA leaves dq in lane groups 0 and 1 and dk in 2
  //       and 3; groups 0 and 2 write);
  //   df: [s][h] x 256 lane partials (the pass sums the whole block, in any
  //       order); fp32 inputs put them at the same offsets within the block
  //       as the qk partials, so that a step's dk and df partials leave in
  //       one ds_write2st64;
  //   dv: [s][h] x [v'][20], the 16 (tile, g) partials of row v' at column
  //       (tile + 4 g + v') mod 16.
  static constexpr int kQKRow = HALF ? 64 : 256;
  static constexpr int kQK = kSub * 2 * HPW * kQKRow;
  static constexpr int kDF = kSub * HPW * 256;
  static constexpr int kDV = kSub * HPW * 320;
  static constexpr int kPart = kQK + kDF + kDV;   // one set, in this order
  // with the gate: alpha, beta of the HPW heads, [h][2], then the dalpha,
  // dbeta sums of each df wave's four lane rows, [wave][row][2]
  static constexpr int kGpar = GATE ? 2 * HPW + HPW * 8 : 0;
  static constexpr int kFloats = kNStage * kBuf + kXpose + kNPart * kPart + kGpar;
  static constexpr int kBytes = kFloats * 4;
};

// Staging of one sub-chunk (kSub steps from t0, the first len of them real)
// through registers into an LDS buffer.  The waves of the last NL roles load:
// thread u of them fetches one 16-byte chunk of q, k, v or u = dy, and one f
// value.  The
// load path is the same straight line for every loading thread (addresses of
// steps past len, of a missing head, and of idle threads are clamped to valid
// data), so no register of an in-flight load is ever merged or copied and
// nothing waits on the loads before they are staged.  Steps past len are
// staged as f = 1, q = k = v = u = 0.
template <typename TIn, int HPW, int NWAVES, bool GATE>
struct BwdStage {
  static constexpr int EPC = 16 / (int)sizeof(TIn);          // elements per chunk
  static constexpr int nQ = kSub * 64 / EPC;                  // q chunks (and k chunks)
  static constexpr int nV = kSub * HPW * 16 / EPC;            // v chunks
  static constexpr int nU = kSub * HPW * 16 / 4;              // dy chunks (fp32)
  static constexpr int nChunks = 2 * nQ + nV + nU;
  static constexpr int NL = (nChunks + 63) / 64;              // loading waves
  static_assert(NL <= NWAVES && kSub * HPW <= 64 * NL, "staging threads");
  u32x4 r;
  TIn fr;

  // chunk u -> kind (0 q, 1 k, 2 v, 3 dy, 4 idle), step t, element offset e0
  // within the step's row (q, k: of 64; v, dy: of the HPW heads' 16 each)
  __device__ static void decode(int u, int& kind, int& t, int& e0) {
    if (u < nQ) { kind = 0; t = u / (64 / EPC); e0 = (u % (64 / EPC)) * EPC; }
    else if (u < 2 * nQ) { u -= nQ; kind = 1; t = u / (64 / EPC); e0 = (u % (64 / EPC)) * EPC; }
    else if (u < 2 * nQ + nV) { u -= 2 * nQ; kind = 2; t = u / (HPW * 16 / EPC); e0 = (u % (HPW * 16 / EPC)) * EPC; }
    else if (u < nChunks) { u -= 2 * nQ + nV; kind = 3; t = u / (HPW * 4); e0 = (u % (HPW * 4)) * 4; }
    else { kind = 4; t = 0; e0 = 0; }
  }

  // rw: the wave's role (role_wave); the last NL roles load
  __device__ void load(const BwdArgs& a, int rw, int lane, int b, int n0, int t0, int len) {
    if (rw < NWAVES - NL) return;
    const int u = (rw - (NWAVES - NL)) * 64 + lane;
    int kind, t, e0;
    decode(u, kind, t, e0);
    const bool ok = t < len && (kind < 2 || n0 + e0 / 16 < a.N);
    const int tt = ok ? t : 0;
    const int ee = ok ? e0 : e0 % 16;                     // a missing head reads head n0
    const size_t row = (size_t)b * a.T + t0 + tt;         // (b, t0 + tt)
    const char* p;
    if (kind == 0) p = (const char*)((const TIn*)a.q + row * 64 + ee);
    else if (kind == 1) p = (const char*)((const TIn*)a.k + row * 64 + ee);
    else if (kind == 2) p = (const char*)((const TIn*)a.v + (row * a.N + n0) * 16 + ee);
    else if (kind == 3) p = (const char*)(a.dy + (row * a.N + n0) * 16 + ee);
    else p = (const char*)((const TIn*)a.q + row * 64);
    r = *(const u32x4*)p;
    // f of (step, head) for threads u < kSub * HPW
    const int ft = u / HPW, fh = u % HPW;
    const bool fok = u < kSub * HPW && ft < len && n0 + fh < a.N;
    const TIn* fsrc = (const TIn*)(GATE ? a.ga : a.f);   // f, or the gate's pre-activation
    fr = fsrc[((size_t)b * a.T + t0 + (fok ? ft : 0)) * a.N + n0 + (fok ? fh : 0)];
  }

  // gpar: alpha, beta of the HPW heads, [h][2] (with the gate)
  // dy is staged multiplied by sig (the gradients' scale)
  __device__ void store(float* buf, int rw, int lane, int n0, int len, int N, const float* gpar, float sig) const {
    if (rw < NWAVES - NL) return;
    float* K_s = buf;
    float* Q_s = K_s + kSub * 64;
    float* V_s = Q_s + kSub * 64;
    float* F_s = V_s + kSub * HPW * 16;
    float* U_s = F_s + kSub * HPW * 4;
    float* Kp_s = U_s + kSub * HPW * 16;
    float* G_s = Kp_s + kSub * 64;
    _Float16* UV_s = (_Float16*)(G_s + (GATE ? kSub * HPW * 2 : 0));   // [s][h][u | v][4][8] fp16
    const int u = (rw - (NWAVES - NL)) * 64 + lane;
    int kind, t, e0;
    decode(u, kind, t, e0);
    const bool ok = t < len && (kind < 2 || n0 + e0 / 16 < N);
    float x[EPC];
    if (kind == 3 || sizeof(TIn) == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r[i] << 16);
        x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
      }
    }
    const int n = kind == 3 ? 4 : EPC;                    // values in this chunk
    if (!ok) {
#pragma unroll
      for (int i = 0; i < EPC; ++i) x[i] = 0.f;
    }
    if (kind == 0) {
#pragma unroll
      for (int i = 0; i < EPC; i += 4) *(f4*)(Q_s + t * 64 + e0 + i) = f4{x[i], x[i + 1], x[i + 2], x[i + 3]};
    } else if (kind == 1) {
      // row e = 16 tile + 4 r + g goes to [tile][g][r] of Kp_s; a chunk starts
      // at a multiple of 4, so element i sits at base + (i % 4) * 4 + i / 4
      if constexpr (sizeof(TIn) == 2) {
        // k itself in fp16 (exact for bf16 values in fp16's normal range); a
        // chunk is 8 rows, r0 and r0 + 1 of each g, which sit side by side
        uint32_t* kp = (uint32_t*)((_Float16*)Kp_s + t * 64 + (e0 / 16) * 16 + (e0 % 16) / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) kp[i * 2] = __builtin_bit_cast(uint32_t, (h2{(_Float16)x[i], (_Float16)x[i + 4]}));
      }
#pragma unroll
      for (int i = 0; i < EPC; ++i) x[i] *= kScale;
#pragma unroll
      for (int i = 0; i < EPC; i += 4) *(f4*)(K_s + t * 64 + e0 + i) = f4{x[i], x[i + 1], x[i + 2], x[i + 3]};
      if constexpr (sizeof(TIn) == 4) {
        float* kp = Kp_s + t * 64 + (e0 / 16) * 16 + (e0 % 16) / 4;   // c k
#pragma unroll
        for (int i = 0; i < EPC; ++i) kp[(i % 4) * 4 + i / 4] = x[i];
      }
    } else if (kind == 2) {
#pragma unroll
      for (int i = 0; i < EPC; i += 4) *(f4*)(V_s + t * HPW * 16 + e0 + i) = f4{x[i], x[i + 1], x[i + 2], x[i + 3]};
      if constexpr (sizeof(TIn) == 2) {
        // v (exact in fp16 in the normal range) in k-slots 4..7 of the v
        // half; a chunk is two lane groups' quads
        _Float16* d = UV_s + t * HPW * 64 + (e0 / 16) * 64 + 32 + ((e0 % 16) / 4) * 8;
        const _Float16 z = (_Float16)0.0f;
        *(h8*)d = h8{z, z, z, z, (_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
        *(h8*)(d + 8) = h8{z, z, z, z, (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]};
      }
    } else if (kind == 3) {
      const f4 us = f4{x[0], x[1], x[2], x[3]} * sig;
      *(f4*)(U_s + t * HPW * 16 + e0) = us;
      if constexpr (sizeof(TIn) == 2) {   // u in k-slots 0..3 of the u half
        const h4 uh = to_half4(us), z = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
        *(h8*)(UV_s + t * HPW * 64 + (e0 / 16) * 64 + ((e0 % 16) / 4) * 8) =
            __builtin_shufflevector(uh, z, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
    (void)n;
    if (u < kSub * HPW) {
      const int ft = u / HPW, fh = u % HPW;
      const bool real = ft < len && n0 + fh < N;
      float ff = 1.0f;
      f2 gf = {0.f, 0.f};
      if (GATE && real) {
        // f = exp(-alpha sp), df/da = -alpha f sigmoid, df/dalpha = -sp f
        const f2 ab = *(const f2*)(gpar + fh * 2);
        const GateVal gv = gate_value(to_f32(fr), ab[0], ab[1]);
        ff = gv.f;
        gf = f2{-ab[0] * gv.f * gv.sig, -gv.sp * gv.f};
      } else if (real) {
        ff = to_f32(fr);
      }
      const float gg = 1.0f - ff;
      *(f4*)(F_s + u * 4) = f4{ff, kScale * gg, -2.0f * kScale * gg, gg};
      if (GATE) *(f2*)(G_s + gate_slot<HPW>(ft, fh) * 2) = gf;
    }
  }
};

// Role of wave w in the reduction pass and in the staging (roles: 0 dq, 1 dk,
// then one dv wave per head, one df wave per four (step, head) pairs, and
// the last NL loaders).  Waves w, w + 4, w + 8 and w + 12 of a workgroup share
// one SIMD (checked on the GPU), and the pass ends at a barrier, so with four
// heads and three loaders the roles are dealt out to even the SIMDs: dq, dk
// and the last head's dv and df on one; a loader, a dv and a df on each other.
template <int HPW, int NL>
__device__ __forceinline__ int role_wave(int w) {
  if constexpr (HPW == 4 && NL == 3) return w == 0 ? 0 : w <= 3 ? 12 + w : w - 3;
  return w;
}

// Accumulator-input variant of the contraction used by the C update:
// returns (W D^T)^T + cin in the transposed frame, i.e. A = W (not W^T).
// bf16 inputs: W (exact in fp16, see m2rnn_device.h) and D rounded once to
// fp16, with D normalised through the scale of dy; each product is then off
// by at most 2^-11 relative, against 2^-8 for a bf16 rounding, which the
// recursion for C amplified past the bf16-input bar.
template <typename TIn> struct WBackOperand;
template <> struct WBackOperand<bf16_t> {
  h4 a;
  __device__ void load(const bf16_t* Wn, int g, int m) {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = (_Float16)(Wn ? to_f32(Wn[m * 16 + 4 * g + s]) : 0.0f);   // W[m][4g + s]
  }
  __device__ f4 apply(f4 d, f4 cin) const { return apply_half(to_half4(d), cin); }
  __device__ f4 apply_half(h4 dh, f4 cin) const { return mfma_f16(a, dh, cin); }
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

// dW[v][v'] += sum over 16 rows kk of A[kk][v] B[kk][v'], with lane (g, m)
// holding A, B at rows 4r + g (r = 0..3) and column m: four exact
// v_mfma_f32_16x16x4_f32 (fp32 inputs; bf16 inputs contract the fp16 tiles
// in one v_mfma_f32_16x16x16_f16, each product then off by at most 2^-10
// relative, independently over rows and time).
__device__ __forceinline__ f4 dw_update(f4 a, f4 b, f4 acc) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], acc, 0, 0, 0);
  return acc;
}

// The rest of one forward step of one tile (no readout) once x = c (H W)^T
// is known: returns r = (1 - tanh)/2 and updates P in place.
__device__ __forceinline__ f4 fwd_tile_finish(f4 x, f4& P, float ck, f4 vv, f4 fc) {
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

// Sum over lanes of four values at once: returns, in every lane of 16-lane
// row r, the sum over all 64 lanes of x[o] with o = 2 (r & 1) + (r >> 1).
// v_permlane32_swap(a, b) yields {[a_lo, b_lo], [a_hi, b_hi]} by 32-lane
// halves and v_permlane16_swap(a, b) yields {[a0, b0, a2, b2], [a1, b1, a3, b3]}
// by 16-lane rows (checked on the GPU).
__device__ __forceinline__ float sum4_over_lanes(float x0, float x1, float x2, float x3) {
  auto s32 = [](float p, float q) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, p), __builtin_bit_cast(uint32_t, q),
                                                    false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  };
  const float y01 = s32(x0, x1);   // lanes 0..31: x0 partial, 32..63: x1 partial
  const float y23 = s32(x2, x3);
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, y01), __builtin_bit_cast(uint32_t, y23),
                                                  false, false);
  // rows: x0, x2, x1, x3, each summed over its four lane groups so far
  return row_sum16(__builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
}

// HS: the restart states are the replay's, c H in fp16 (bf16 inputs);
// otherwise H in fp32 (the caller's checkpoints, or the replay's c H for fp32
// inputs), scaled by a.ck_scale.
template <typename TIn, int HPW, bool GATE, bool HS>
__global__ __launch_bounds__(256 * HPW) __attribute__((amdgpu_waves_per_eu(4))) void m2rnn_bwd_kernel(BwdArgs a) {
  // bf16 inputs: fp16 LDS transposes, dv partials from k itself; fp32
  // inputs: fp32 transposes, dv partials from c k
  constexpr bool kHalf = sizeof(TIn) == 2;
  static_assert(kHalf || !HS, "fp16 restart states are for bf16 inputs");
  typedef BwdCfg<HPW, GATE, kHalf> Cfg;
  constexpr float kDvScale = kHalf ? 1.0f : kInvScale;
  extern __shared__ float smem[];
  float* xpose = smem + Cfg::kNStage * Cfg::kBuf;
  float* parts = xpose + Cfg::kXpose;   // kNPart sets of {qk, df, dv} partials

  const int tid = threadIdx.x;
  // wave-uniform indices live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, g = lane / 16, m = lane % 16;
  const int hw = w / 4, j = w % 4;               // head in group, row tile
  typedef BwdStage<TIn, HPW, Cfg::NWAVES, GATE> Stage;
  const int rw = role_wave<HPW, Stage::NL>(w);   // role in the pass and the staging
  const int ngroups = (a.N + HPW - 1) / HPW;
  const int b = blockIdx.x / ngroups;
  const int grp = blockIdx.x % ngroups;
  const int n0 = grp * HPW;
  const int n = n0 + hw;
  const bool live = n < a.N;
  const int kk = 16 * j + m;                      // this lane's state row
  float* xp = xpose + w * Cfg::kXw;
  const size_t head = (size_t)b * a.N + n;
  // stored states H at t = s * L (s = 0 .. ns-1), L = a.ckpt_every <= kSub
  const int L = a.ckpt_every, ns = a.nck;
  const float* Hs = a.H_ckpt + head * (size_t)ns * 1024 + kk * 16 + 4 * g;
  const _Float16* Hh = (const _Float16*)a.H_ckpt + head * (size_t)ns * 1024 + kk * 16 + 4 * g;   // HS
  // this lane's slots in the partials blocks (see BwdCfg).  bf16 inputs:
  // lane group 0 writes row kk of the dq, dk blocks, and the df partial of
  // lane group g sits in its quarter of the block rotated by 16 (g & 1) rows,
  // so the two groups that share a write cycle hit different banks.
  const int qk_slot = kHalf ? hw * 64 + kk : hw * 256 + g * 64 + (((4 * j + m / 4 + 4 * g) & 15) << 2) + (m & 3);
  const int df_slot = kHalf ? hw * 256 + g * 64 + ((kk + 16 * (g & 1)) & 63) : qk_slot;
  const int qk2_slot = (g >> 1) * HPW * 64 + qk_slot;   // bf16: dq (groups 0, 1) or dk (2, 3)
  const int dv_slot = hw * 320 + m * 20 + ((j + 4 * g + m) & 15);

  typename ReplayOperand<TIn>::type Af;
  Af.load(live ? (const TIn*)a.W + (size_t)n * 256 : nullptr, g, m);
  WBackOperand<TIn> Ab;
  Ab.load(live ? (const TIn*)a.W + (size_t)n * 256 : nullptr, g, m);

  // the gradients' scale: dy and dH_T enter multiplied by sig, every output
  // leaves multiplied by isig (each wave reduces the partial maxima itself)
  float sig = 1.0f, isig = 1.0f;
  if (a.ws_amax) {
    float mx = 0.0f;
    for (int i = lane; i < kAmaxParts; i += 64) mx = fmaxf(mx, a.ws_amax[i]);
    grad_scale(wave_max(mx), sig, isig);
    sig = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sig)));   // uniform
    isig = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, isig)));
  }
  // C in the transposed frame: lane (g, m), register i = C[kk][4g + i]
  f4 C = {0.f, 0.f, 0.f, 0.f};
  if (live && a.dH_T) C = *(const f4*)(a.dH_T + head * 1024 + kk * 16 + 4 * g) * sig;
  f4 dW = {0.f, 0.f, 0.f, 0.f};   // lane (g, m), register i: c * dW[4g + i][m] partial
  // dv waves (one per head): w_r of their (head, v') and the dw_r partial of
  // their step slot
  const bool dv_wave = rw >= Cfg::kDvWave && rw < Cfg::kDvWave + HPW;
  float wr_e = 0.f, dwr = 0.f;
  // the gate parameters of the group's heads, read by the threads that stage
  // f; the df waves' dalpha, dbeta sums (slot gate_slot(s, h): row r of df
  // wave d accumulates its (step, head) pair over the sub-chunks)
  float* gpar = parts + Cfg::kNPart * Cfg::kPart;
  float* gacc = gpar + 2 * HPW;
  if (GATE) {
    if (tid < HPW) {
      const bool ok = n0 + tid < a.N;
      gpar[tid * 2] = ok ? to_f32(((const TIn*)a.galpha)[n0 + tid]) : 0.f;
      gpar[tid * 2 + 1] = ok ? to_f32(((const TIn*)a.gbeta)[n0 + tid]) : 0.f;
    }
    if (tid < HPW * 8) gacc[tid] = 0.f;
    __syncthreads();
  }
  constexpr bool gate = GATE;
  if (dv_wave) {
    const int hh = rw - Cfg::kDvWave;
    if (n0 + hh < a.N) wr_e = to_f32(((const TIn*)a.wr)[(size_t)(n0 + hh) * 16 + m]);
  }
  if (!live) {
    // a missing head adds zero to the dq, dk sums of the pass
    // (bf16 inputs: every lane group writes group 0's zero)
#pragma unroll
    for (int ps = 0; ps < Cfg::kNPart; ++ps)
#pragma unroll
      for (int s = 0; s < 2 * kSub; ++s) parts[ps * Cfg::kPart + s * HPW * Cfg::kQKRow + qk_slot] = 0.f;
  }

  // stage the first kNStage - 1 sub-chunks (the latest); one that does not
  // exist stages sub-chunk 0 into a buffer no one reads
#pragma unroll
  for (int i = 0; i < Cfg::kNStage - 1; ++i) {
    Stage st;
    const int t0 = max(ns - 1 - i, 0) * L, len0 = min(L, a.T - t0);
    st.load(a, rw, lane, b, n0, t0, len0);
    st.store(smem + i * Cfg::kBuf, rw, lane, n0, len0, a.N, gpar, sig);
  }
  // the next restart state, prefetched one sub-chunk ahead and scaled by c
  // only when it is used (so nothing waits on the load early)
  f4 Hnext = {0.f, 0.f, 0.f, 0.f};
  h4 Hnext_h = {};
  if constexpr (HS) {
    if (live) Hnext_h = *(const h4*)(Hh + (size_t)(ns - 1) * 1024);
  } else {
    if (live) Hnext = *(const f4*)(Hs + (size_t)(ns - 1) * 1024);
  }
  __syncthreads();

  // Wave priorities.  The four waves of a SIMD run the same dependent chains
  // from the same barrier, and issue goes to the oldest ready wave, so
  // without them the youngest wave finishes its replay last and runs its
  // reverse sweep almost alone while the others wait at the barrier.  Each
  // wave lowers its priority as it advances through the sub-chunk (3, 3, 2,
  // 2 over the replay's steps, 2, 1, 1, 0 over the reverse steps), which
  // hands the issue slots to the waves behind and keeps the four together;
  // in the pass the loaders, whose staging store is its longest path, take
  // priority 3 and the other roles 1.
  for (int sb = ns - 1, it = 0; sb >= 0; --sb, ++it) {
    __builtin_amdgcn_s_setprio(3);
    const int t0 = sb * L, len = min(L, a.T - t0);
    f4 P;
    const h4 P0h = Hnext_h;   // HS: the restart state as stored, c H in fp16
    if constexpr (HS) P = __builtin_convertvector(P0h, f4);
    else P = Hnext * a.ck_scale;
    // prefetch the sub-chunk this pass stages, kNStage - 1 ahead (registers
    // live for this iteration only), and the next restart state.  Near the
    // end sub-chunk 0 is fetched again and staged into a buffer no one reads:
    // no branch, so nothing in flight gets copied.
    const int sn = max(sb - (Cfg::kNStage - 1), 0), sr = sb > 0 ? sb - 1 : 0;
    Stage st;
    const int lenn = min(L, a.T - sn * L);
    st.load(a, rw, lane, b, n0, sn * L, lenn);
    if constexpr (HS) {
      if (live) Hnext_h = *(const h4*)(Hh + (size_t)sr * 1024);
    } else {
      if (live) Hnext = *(const f4*)(Hs + (size_t)sr * 1024);
    }
    const float* buf = smem + (it % Cfg::kNStage) * Cfg::kBuf;
    float* qkbuf = parts + (it % Cfg::kNPart) * Cfg::kPart;
    float* dfbuf = qkbuf + Cfg::kQK;
    float* dvbuf = dfbuf + Cfg::kDF;
    const float* K_s = buf;
    const float* Q_s = K_s + kSub * 64;
    const float* V_s = Q_s + kSub * 64;
    const float* F_s = V_s + kSub * HPW * 16;
    const float* U_s = F_s + kSub * HPW * 4;
    const float* Kp_s = U_s + kSub * HPW * 16;     // k permuted, [s][tile][g][r] (c k in fp32, k in fp16)
    const float* G_s = Kp_s + kSub * 64;            // gate factors, [df wave][row][2]
    const _Float16* UV_s = (const _Float16*)(G_s + (GATE ? kSub * HPW * 2 : 0));   // dq, dk A operand

    if (live) {
      // replay the sub-chunk keeping H_{t-1} and Z_t on chip (and, for bf16
      // inputs, the fp16 rounding of H_{t-1} its contraction used)
      f4 Pp[kSub], Z[kSub];
      // 1 / c in an SGPR: a VOP3 instruction (which has the negation
      // modifier) takes no literal constant on this target
      float kis = kInvScale;
      asm volatile("" : "+s"(kis));
      h4 Ph[kSub + 1];   // bf16 inputs: the fp16 states, H_t of the last step included
      // dq_t[kk] (this head) = sum_v H_t[kk][v] u_t[v] = (1/c) sum_v P u:
      // fp32 inputs, per-lane partials over the lane's four v in the replay;
      // bf16 inputs, in the reverse sweep together with dk (below)
      // Steps s >= len of a short last sub-chunk are staged as f = 1 with
      // q = k = v = u = 0: an exact identity for C and a zero contribution to
      // dq, dk, dv, dW and dw_r (df of such steps is not stored), so all kSub
      // steps run unguarded.
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        if (s < 2) __builtin_amdgcn_s_setprio(3);
        else __builtin_amdgcn_s_setprio(2);
        {
          const f4 vv = *(const f4*)(V_s + (s * HPW + hw) * 16 + 4 * g);
          const f4 fc = *(const f4*)(F_s + (s * HPW + hw) * 4);
          Pp[s] = P;
          f4 x;
          if constexpr (kHalf) {
            Ph[s] = HS && s == 0 ? P0h : to_half4(P);   // (P0h is exactly P in fp16)
            x = Af.times_half(Ph[s]);
          } else {
            x = Af.times_state(P);
          }
          const f4 r = fwd_tile_finish(x, P, K_s[s * 64 + kk], vv, fc);
#pragma unroll
          for (int i = 0; i < 4; ++i) Z[s][i] = fmaf(-2.0f, r[i], 1.0f);
          if constexpr (kHalf) {
            // bf16 inputs keep H_{t-1} - Z for df in place of H_{t-1} (the
            // transposes take the fp16 state)
#pragma unroll
            for (int i = 0; i < 4; ++i) Pp[s][i] = fmaf(Pp[s][i], kis, -Z[s][i]);
          }
          if constexpr (!kHalf) {
            const f4 uu = *(const f4*)(U_s + (s * HPW + hw) * 16 + 4 * g);
            float dq = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) dq = fmaf(P[i], uu[i], dq);
            qkbuf[(2 * s) * HPW * Cfg::kQKRow + qk_slot] = dq;
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep each step's loads in its step
      }
      if constexpr (kHalf) Ph[kSub] = to_half4(P);
      // reverse sweep over the sub-chunk.  The dW / dv contractions over the
      // tile's rows read H_{t-1} and D back from LDS in MFMA operand layout;
      // they run one step behind the sweep so that the LDS round trip
      // overlaps the next step's arithmetic (LDS requests of a wave complete
      // in issue order, so no wait is needed between the write and the read).
      //
      // bf16 inputs: the fp16 tiles the contractions already rounded go to
      // LDS as 8-byte chunks (lane (g, m): row m, columns 4g..4g+3) and come
      // back with ds_read_b64_tr_b16, which hands lane i of each 16-lane
      // group, as element s, element i % 4 of the chunk that lane
      // 4 s + i / 4 of the group addressed (checked on the GPU).  Lane (g, m)
      // addresses the chunk (row 4 (m / 4) + g, columns 4 (m % 4) ..), so it
      // receives X[4 s + g][m], s = 0..3: the operand layout.  Chunk (row,
      // block) of a tile sits at 16 (row / 4) + 4 ((row % 4) ^ block) +
      // (block ^ row / 4), which spreads the 16 chunks of every 16-lane
      // write and every 16-lane transposed read over distinct banks.
      const int xw = 16 * (m >> 2) + 4 * ((m & 3) ^ g) + (g ^ (m >> 2));            // chunk this lane writes
      const int xr = 16 * (m >> 2) + 4 * (g ^ (m & 3)) + ((m & 3) ^ (m >> 2));        // chunk it reads
      h4* xh = (h4*)xp;   // [slot][H | D][64 chunks]
      auto drain = [&](int ps) {
        if constexpr (kHalf) {
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const h4 ah = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_i16x4*)(xh + (ps & 1) * 128 + xr)));   // c H_{t-1}[16j+4s+g][m]
          const h4 bh = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_i16x4*)(xh + (ps & 1) * 128 + 64 + xr)));   // D[16j+4s+g][m]
          const h4 kh = *(const h4*)((const _Float16*)Kp_s + ps * 64 + j * 16 + g * 4);   // k[16j+4s+g]
          const float dvp = __builtin_amdgcn_fdot2(h2{bh[0], bh[1]}, h2{kh[0], kh[1]},
                                                   __builtin_amdgcn_fdot2(h2{bh[2], bh[3]}, h2{kh[2], kh[3]}, 0.0f, false),
                                                   false);
          dW = mfma_f16(ah, bh, dW);
          dvbuf[ps * HPW * 320 + dv_slot] = dvp;            // partial of dv[v' = m] over rows 4s+g
        } else {
          const float* xs = xp + (ps & 1) * 2 * Cfg::kTile;
          const f4 ckp = *(const f4*)(Kp_s + ps * 64 + j * 16 + g * 4);   // c k[16j+4r+g], r = 0..3
          float dvp = 0.f;
          f4 av, bv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int at = (m / 4) * Cfg::kXs + (4 * r + g) * 4 + m % 4;
            av[r] = xs[at];                                   // c H_{t-1}[16j+4r+g][v = m]
            bv[r] = xs[Cfg::kTile + at];                      // D[16j+4r+g][v' = m]
            dvp = fmaf(bv[r], ckp[r], dvp);
          }
          dW = dw_update(av, bv, dW);
          dvbuf[ps * HPW * 320 + dv_slot] = dvp;              // partial of dv[v' = m] over rows 4r+g
        }
      };
#pragma unroll
      for (int s = kSub - 1; s >= 0; --s) {
        if (s == kSub - 1) __builtin_amdgcn_s_setprio(2);
        else if (s > 0) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        {
          const f4 fc = *(const f4*)(F_s + (s * HPW + hw) * 4);   // f, c(1-f), -2c(1-f), 1-f
          const f4 uu = *(const f4*)(U_s + (s * HPW + hw) * 16 + 4 * g);
          const float qv = Q_s[s * 64 + kk];
          f4 R, D, fR;
          float dfp = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            R[i] = fmaf(qv, uu[i], C[i]);                            // R = C + q u^T
            const float gz = fc[3] * Z[s][i];
            D[i] = R[i] * fmaf(-gz, Z[s][i], fc[3]);                 // (1-f) R (1 - Z^2)
            dfp = fmaf(R[i], kHalf ? Pp[s][i] : fmaf(Pp[s][i], kInvScale, -Z[s][i]), dfp);   // <R, H_{t-1} - Z>
            fR[i] = fc[0] * R[i];
          }
          // dk_t[kk] (this head) = sum_v' D[kk][v'] v_t[v'] and the per-lane
          // partial of df_t
          float* pf = dfbuf + s * HPW * 256 + df_slot;
          // C_{t-1} = f R + D W^T; stage H_{t-1} and D of this step, finish
          // the previous step
          if constexpr (kHalf) {
            const h4 Dh = to_half4(D);
            C = Ab.apply_half(Dh, fR);
            // dq_t and dk_t in one MFMA (a 16-deep product costs a 32-deep
            // one's cycles): A rows 0..7 hold u in k-slots 0..3 of each lane
            // group, rows 8..15 v in k-slots 4..7; B holds H_t (the next
            // step's fp16 state) in slots 0..3 and D in 4..7.  Result rows
            // 0..7 are dq[kk], rows 8..15 dk[kk]; lane groups 0 and 2 write.
            const h8 uv = *(const h8*)(UV_s + (s * HPW + hw) * 64 + (m >> 3) * 32 + 8 * g);
            const f4 qk = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                uv, __builtin_shufflevector(Ph[s + 1], Dh, 0, 1, 2, 3, 4, 5, 6, 7), f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            if ((g & 1) == 0) qkbuf[2 * s * HPW * 64 + qk2_slot] = qk[0];
            *pf = dfp;
            xh[(s & 1) * 128 + xw] = Ph[s];
            xh[(s & 1) * 128 + 64 + xw] = Dh;
          } else {
            const f4 vv = *(const f4*)(V_s + (s * HPW + hw) * 16 + 4 * g);
            float dk = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) dk = fmaf(D[i], vv[i], dk);
            qkbuf[(2 * s + 1) * HPW * Cfg::kQKRow + qk_slot] = dk;
            *pf = dfp;
            C = Ab.apply(D, fR);
            *(f4*)(xp + (s & 1) * 2 * Cfg::kTile + g * Cfg::kXs + m * 4) = Pp[s];
            *(f4*)(xp + (s & 1) * 2 * Cfg::kTile + Cfg::kTile + g * Cfg::kXs + m * 4) = D;
          }
          if (s < kSub - 1) drain(s + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      drain(0);
    }
    __syncthreads();
    if (rw >= Cfg::NWAVES - Stage::NL) __builtin_amdgcn_s_setprio(3);
    else __builtin_amdgcn_s_setprio(1);
    // ---- pass: reduce this sub-chunk's partials; each wave has one role.
    if (rw < 2) {
      // dq (wave 0), dk (wave 1): lane (s, 4-row quad r4) sums the HPW heads
      // and four lane groups -> workspace [b][grp][t][dq | dk][64]
      const int s = lane / 16, r4 = lane % 16;
      const float* src = qkbuf + (2 * s + rw) * HPW * Cfg::kQKRow;
      // bf16: lane group 0's copy of the whole sum per head; fp32: four
      // lane-group partials per head.  The sum starts from the first term.
      constexpr int kParts = kHalf ? 1 : 4;
      auto part = [&](int hh, int gg) {
        return kHalf ? *(const f4*)(src + hh * 64 + 4 * r4)
                     : *(const f4*)(src + hh * 256 + gg * 64 + (((r4 + 4 * gg) & 15) << 2));
      };
      f4 acc = part(0, 0);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
        for (int gg = 0; gg < kParts; ++gg)
          if (hh + gg > 0) acc += part(hh, gg);
      }
      acc *= rw == 0 ? kInvScale * isig : isig;
      float* dst = a.ws_dqk + (((size_t)b * ngroups + grp) * a.T + t0) * 128;   // uniform
      if (s < len) *(f4*)(dst + (unsigned)(s * 128 + rw * 64 + 4 * r4)) = acc;
    } else if (dv_wave) {
      // dv[b][t][n][v'] = (1/c) (sum of the 16 (tile, g) partials) + w_r u; dw_r
      const int hh = rw - Cfg::kDvWave, s = lane / 16, e = lane % 16;
      const float* d = dvbuf + (s * HPW + hh) * 320 + e * 20;
      const f4 p = (*(const f4*)d + *(const f4*)(d + 4)) + (*(const f4*)(d + 8) + *(const f4*)(d + 12));
      const float uu = U_s[(s * HPW + hh) * 16 + e];
      dwr = fmaf(uu, V_s[(s * HPW + hh) * 16 + e], dwr);
      float* dst = a.dv + (((size_t)b * a.T + t0) * a.N + n0) * 16;   // uniform
      if (s < len && n0 + hh < a.N)
        dst[(unsigned)((s * a.N + hh) * 16 + e)] = fmaf(wr_e, uu, ((p[0] + p[1]) + (p[2] + p[3])) * kDvScale) * isig;
    } else if (rw < Cfg::kRoleWaves) {
      // df[b][t][n]: wave d sums the pairs p = 4 d + o (p = step HPW + head)
      const int d = rw - Cfg::kDfWave;
      float x[4];
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const f4 p = *(const f4*)(dfbuf + (4 * d + o) * 256 + lane * 4);
        x[o] = (p[0] + p[1]) + (p[2] + p[3]);
      }
      const float tot = sum4_over_lanes(x[0], x[1], x[2], x[3]) * isig;   // row g: x[2 (g & 1) + (g >> 1)]
      const int pg = 4 * d + 2 * (g & 1) + (g >> 1), s = pg / HPW, hh = pg % HPW;
      float out = tot;
      if (gate) {
        // chain rule through f = exp(-alpha softplus(a + beta)): da, and the
        // per-head sums for dalpha, dbeta
        const f2 gf = *(const f2*)(G_s + (d * 4 + g) * 2);
        out = tot * gf[0];
        if (m == 0 && s < len && n0 + hh < a.N) {
          f2* acc = (f2*)(gacc + (d * 4 + g) * 2);   // this lane's own slot
          *acc = *acc + f2{tot * gf[1], out};
        }
      }
      float* dst = a.df + ((size_t)b * a.T + t0) * a.N + n0;   // uniform
      if (GATE) dst = sgpr_ptr(dst);
      if (m == 0 && s < len && n0 + hh < a.N) dst[(unsigned)(s * a.N + hh)] = out;
    }
    st.store(smem + ((it + Cfg::kNStage - 1) % Cfg::kNStage) * Cfg::kBuf, rw, lane, n0, lenn, a.N, gpar, sig);
    if (Cfg::kNPart == 1) __syncthreads();
  }
  if (Cfg::kNPart > 1) __syncthreads();   // every pass has ended

  if (live) {
    float* dst = a.ws_dW + (head * 4 + j) * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * g + i) * 16 + m] = dW[i] * (kInvScale * isig);
    // the recursion for C ends at C_0 = dL/dH_0
    if (a.dH_0) *(f4*)(a.dH_0 + head * 1024 + kk * 16 + 4 * g) = C * isig;
  }
  // dw_r: the dv waves hold one partial per (step slot, head, v'); sum the
  // step slots in a fixed order
  float* dwr_s = parts + Cfg::kQK;   // the first set's df partials, free now
  if (dv_wave) dwr_s[(rw - Cfg::kDvWave) * 64 + lane] = dwr;
  __syncthreads();
  if (w == 0 && lane < HPW * 16) {
    const int hh = lane / 16, e = lane % 16;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < kSub; ++s) acc += dwr_s[hh * 64 + s * 16 + e];
    if (n0 + hh < a.N) a.ws_dwr[((size_t)b * a.N + n0 + hh) * 16 + e] = acc * isig;
  }
  if (gate && w == 1 && lane < HPW && n0 + lane < a.N) {
    const int hh = lane;
    f2 acc = {0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSub; ++s) acc += *(const f2*)(gacc + gate_slot<HPW>(s, hh) * 2);
    *(f2*)(a.ws_dgate + ((size_t)b * a.N + n0 + hh) * 2) = acc;
  }
}

// The gradient scale's partial maxima (grad_absmax_part, m2rnn_device.h) as
// a launch of its own, when no chunk replay runs that could carry them.
__global__ __launch_bounds__(256) void m2rnn_bwd_absmax_kernel(const float* dy, size_t ndy4, const float* dH,
                                                              size_t ndh4, float* part) {
  __shared__ float wm[4];
  grad_absmax_part(dy, ndy4, dH, ndh4, part, (int)blockIdx.x, (int)gridDim.x, wm);
}

// Fixed-order sums over workgroups of the dq, dk partials.
__global__ void m2rnn_bwd_reduce_qk_kernel(BwdArgs a) {
  const size_t nqk = (size_t)a.B * a.T * 32;   // float4 groups of dq and dk
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < nqk; u += (size_t)gridDim.x * blockDim.x) {
    const size_t bt = u / 32;
    const int e = (int)(u % 32) * 4;
    const size_t b = bt / a.T, t = bt % a.T;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int gp = 0; gp < a.ngroups; ++gp) acc += *(const f4*)(a.ws_dqk + ((b * a.ngroups + gp) * a.T + t) * 128 + e);
    float* dst = e < 64 ? a.dq + bt * 64 + e : a.dk + bt * 64 + (e - 64);
    *(f4*)dst = acc;
  }
}

// Per-head sums over batch rows (and row tiles) of the dW, dw_r and gate
// partials, one workgroup per head.  Thread (jt, c) of the first 256 sums the
// dW partials of row tile jt, column group c over the batch rows (b
// ascending, in four interleaved accumulators so that the loads overlap);
// the four row tiles are then added in order.  dw_r and the gate sums use 16
// interleaved lanes per value the same way.
__global__ __launch_bounds__(256) void m2rnn_bwd_reduce_head_kernel(BwdArgs a) {
  __shared__ f4 tiles[4][64];
  __shared__ f4 wr[16][4];
  __shared__ f2 gt[16];
  const int n = blockIdx.x, tid = threadIdx.x;
  {
    const int jt = tid / 64, c = tid % 64;
    f4 acc[4] = {};
    int b = 0;
    for (; b + 3 < a.B; b += 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] += *(const f4*)(a.ws_dW + (((size_t)(b + q) * a.N + n) * 4 + jt) * 256 + c * 4);
    }
    for (int q = 0; b < a.B; ++b, ++q) acc[q] += *(const f4*)(a.ws_dW + (((size_t)b * a.N + n) * 4 + jt) * 256 + c * 4);
    tiles[jt][c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  if (tid < 64) {
    // dw_r: lane l (of 16) sums batch rows b = l, l + 16, ... of column group cg
    const int l = tid / 4, cg = tid % 4;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = l; b < a.B; b += 16) acc += *(const f4*)(a.ws_dwr + ((size_t)b * a.N + n) * 16 + cg * 4);
    wr[l][cg] = acc;
  } else if (a.ga && tid < 80) {
    const int l = tid - 64;
    f2 acc = {0.f, 0.f};
    for (int b = l; b < a.B; b += 16) acc += *(const f2*)(a.ws_dgate + ((size_t)b * a.N + n) * 2);
    gt[l] = acc;
  }
  __syncthreads();
  if (tid < 64) *(f4*)(a.dW + (size_t)n * 256 + tid * 4) = (tiles[0][tid] + tiles[1][tid]) + (tiles[2][tid] + tiles[3][tid]);
  if (tid < 4) {
    f4 acc = wr[0][tid];
#pragma unroll
    for (int l = 1; l < 16; ++l) acc += wr[l][tid];
    *(f4*)(a.dw_r + (size_t)n * 16 + tid * 4) = acc;
  }
  if (a.ga && tid == 0) {
    f2 acc = gt[0];
#pragma unroll
    for (int l = 1; l < 16; ++l) acc += gt[l];
    a.dalpha[n] = acc[0];
    a.dbeta[n] = acc[1];
  }
}

// Heads per workgroup of the sweep by the number of (batch row, head)
// chains: four heads (16 waves, one workgroup per CU) issue the fewest
// instructions per head-step, but need B N / 4 >= 256 workgroups to fill
// the GPU; with fewer chains, two heads or one head per workgroup put each
// chain's four waves on more CUs.
static int bwd_heads_per_group(int B, int N) {
  const long long chains = (long long)B * N;
  return chains >= 1024 ? 4 : chains >= 512 ? 2 : 1;
}

size_t backward_workspace_floats(int B, int T, int N, int ckpt_every, size_t* off_dense, size_t* off_dqk,
                                 size_t* off_dW, size_t* off_dwr, size_t* off_dgate, size_t* off_amax,
                                 int* ngroups) {
  const int hpw = bwd_heads_per_group(B, N);
  const int ng = (int)(((long long)N + hpw - 1) / hpw);
  auto up = [](size_t x) { return (x + 63) & ~(size_t)63; };   // 256-byte aligned regions
  size_t o = 0;
  *off_dense = o;
  if (ckpt_every > kSub) o += up((size_t)B * N * (((size_t)T + kSub - 1) / kSub) * 1024);
  *off_dqk = o;  o += up((size_t)B * ng * T * 128);
  *off_dW = o;   o += up((size_t)B * N * 4 * 256);
  *off_dwr = o;  o += up((size_t)B * N * 16);
  *off_dgate = o; o += up((size_t)B * N * 2);
  *off_amax = o; o += up(kAmaxParts);
  *ngroups = ng;
  return o;
}

// The sweep's dynamic LDS exceeds the default limit, so its kernel takes the
// attribute that allows it, once per device (with that device current) and
// kernel instance; later launches on that device find it set.
constexpr int kMaxDevices = 64;

template <typename TIn, int HPW, bool GATE, bool HS>
static hipError_t set_lds_attribute(hipStream_t stream) {
  static std::mutex mu;
  static bool done[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (done[dev]) return hipSuccess;
  int cur = -1;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)m2rnn_bwd_kernel<TIn, HPW, GATE, HS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          BwdCfg<HPW, GATE, sizeof(TIn) == 2>::kBytes);
  const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
  if (e != hipSuccess) return e;
  if (e2 != hipSuccess) return e2;
  done[dev] = true;
  return hipSuccess;
}

template <typename TIn, int HPW, bool GATE, bool HS>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  typedef BwdCfg<HPW, GATE, sizeof(TIn) == 2> Cfg;
  static_assert(Cfg::kBytes <= 160 * 1024, "backward LDS budget");
  const hipError_t attr = set_lds_attribute<TIn, HPW, GATE, HS>(stream);
  if (attr != hipSuccess) return attr;
  dim3 grid((unsigned)(a.B * a.ngroups)), block(Cfg::NT);
  hipLaunchKernelGGL((m2rnn_bwd_kernel<TIn, HPW, GATE, HS>), grid, block, Cfg::kBytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t blocks = ((size_t)a.B * a.T * 32 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(m2rnn_bwd_reduce_qk_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(m2rnn_bwd_reduce_head_kernel, dim3((unsigned)a.N), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename TIn, bool GATE, bool HS>
static hipError_t launch_bwd_shape(const BwdArgs& a, hipStream_t stream) {
  switch (bwd_heads_per_group(a.B, a.N)) {
    case 4: return launch_bwd_t<TIn, 4, GATE, HS>(a, stream);
    case 2: return launch_bwd_t<TIn, 2, GATE, HS>(a, stream);
    default: return launch_bwd_t<TIn, 1, GATE, HS>(a, stream);
  }
}

hipError_t launch_backward(const BwdArgs& a0, const FwdArgs& replay0, int dtype, hipStream_t stream) {
  BwdArgs a = a0;
  FwdArgs replay = replay0;
  const bool replayed = a.ckpt_every > kSub;
  // The gradients' scale (bf16 inputs; exact fp32 contractions need none):
  // the first kAmaxParts workgroups of the chunk replay when there is one,
  // so that the pass over dy runs beside the replay's arithmetic, else a
  // launch of its own.
  if (dtype == 0) {
    a.ws_amax = nullptr;
  } else {
    const size_t ndy4 = (size_t)a.B * a.T * a.N * 4, ndh4 = a.dH_T ? (size_t)a.B * a.N * 256 : (size_t)0;
    if (replayed) {
      replay.amax_dy = a.dy;
      replay.amax_ndy4 = ndy4;
      replay.amax_dH = a.dH_T;
      replay.amax_ndh4 = ndh4;
      replay.amax_part = a.ws_amax;
      replay.amax_wgs = kAmaxParts;
    } else {
      hipLaunchKernelGGL(m2rnn_bwd_absmax_kernel, dim3(kAmaxParts), dim3(256), 0, stream, a.dy, ndy4, a.dH_T, ndh4,
                         a.ws_amax);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (replayed) {
    // states every kSub steps, replayed from the caller's checkpoints (c H,
    // in fp16 for bf16 inputs)
    hipError_t e = launch_densify(replay, dtype, stream);
    if (e != hipSuccess) return e;
    a.H_ckpt = replay.H_ckpt;
    a.ck_scale = 1.0f;   // the replay stores c H
    a.ckpt_every = kSub;
    a.nck = (a.T + kSub - 1) / kSub;
  }
  if (dtype == 0) return a.ga ? launch_bwd_shape<float, true, false>(a, stream) : launch_bwd_shape<float, false, false>(a, stream);
  if (replayed)
    return a.ga ? launch_bwd_shape<bf16_t, true, true>(a, stream) : launch_bwd_shape<bf16_t, false, true>(a, stream);
  return a.ga ? launch_bwd_shape<bf16_t, true, false>(a, stream) : launch_bwd_shape<bf16_t, false, false>(a, stream);
}

int backward_sub_steps() { return kSub; }

}  // namespace m2rnn

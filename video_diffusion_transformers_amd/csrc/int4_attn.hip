// K2: RotateAttention's INT4 FlashAttention forward on gfx950.
//
// RotateAttention page ("RotateAttention: RoPE-Aware Rotation and Range
// Rectification for INT4 Quantized Attention in Video Generation", Abstract):
// quantized FlashAttention over INT4 Q/K/V, where P = exp(S - max S) is
// non-negative and is quantized to the full unsigned 4-bit range with a fixed
// scale (1/15) and zero point (0) -- "range-optimized P quantization".
//
// What one work-group computes (4 waves x 32 queries = one 128-query block of
// one head; the block shares one Q scale):
//   for each 128-key tile t (ascending):
//     S^T  = K_t Q^T (exact integers I)
//     m'   = max(m, fl(max_j I * c_t)),  c_t = fl(q_scale_l2 * k_scale_t)
//     code = rne(15 * 2^(fl(fl(I*c_t) - m')))            (u4, exact, see below)
//     l    = 2^(m-m') l + sum_j 15 * 2^(...)             (fp32, unquantized;
//            the code-sum variant adds the codes instead)
//     O^T  = 2^(m-m') O^T + v_scale_t * (V_t^T P^T)      (exact integers V.P)
//   O = O / l  -> fp16.
// Two implementations with the same integers:
//  * Int4F8Kernel (production, FP8 layout): Q/K/V codes are the FP8 E4M3
//    bytes of the integers and S^T = K Q^T runs on the 32x32x64 f8f6f4 MFMA,
//    whose fp32 accumulators hold the integer sums exactly.  The P codes enter
//    V^T P^T as FP6 E2M3 values code/2 (every half-integer 0..7.5 is exact in
//    E2M3), converted 32 at a time; the FP8 x FP6 product runs at the FP8
//    rate and its fp32 result is PV/2 exactly.  O is kept in units of the
//    current V block scale.
//  * Int4Kernel (PACKED layout): two codes per byte, unpacked to 16*code in
//    int8 lanes for v_mfma_i32_32x32x32_i8 (the int32 result is 256*I).
// Computing S^T (keys as MFMA rows) leaves every lane holding one query's
// scores in exactly the operand layout the P.V MFMA needs for P^T, so the
// requantized codes never leave registers; the running max, sum and O rows of
// a query live in the same lane pair (lane, lane^32).
//
// P codes, exactly.  The fast path computes y = v_exp_f32(fma(I, c_t,
// log2(15) - m')) ~ 15*2^x and rounds it to nearest even.  |y - 15*2^x| is
// bounded by the rounding of the fused argument (at most ~ulp(|m'| + 8) +
// 2^-21 in x; a wave whose running max is too large for that bound to be
// useful takes the argument from fl(fl(I*c_t) - m') instead) and the exp
// error (< 1 ulp); whenever some y of a 32-key subtile lies within delta of a
// half-integer, that register is recomputed exactly against the thresholds
// tau_k (code = #{k : fl(fl(I*c_t) - m') >= tau_k}).  The self-test entry
// points run the same device functions over every float32 score and over
// random integer scores.
#include <math.h>

#include <type_traits>

#include "rotattn_internal.h"

namespace rotattn {

constexpr int kThreads = 256;
constexpr int kVStride = 144;   // V^T tile row: 128 keys + 16 bytes of padding

struct CodeCtx {
  float iscale;  // exact factor from the incoming score to I (2^-8 on i8 MFMA, 1 on fp8)
  float cq;      // c_t * iscale
  float m15n;    // fl(log2(15)) - m'
  float ct;      // c_t
  float mnew;    // m'
  float delta;   // half-width of the band around each half-integer that takes the exact path
  float l2_15;   // fl(log2(15))
  bool exact_arg;   // wave-uniform: the argument is x + log2(15) with x = fl(fl(I c_t) - m')
};

__device__ __forceinline__ float ulp_pos(float v) {   // ulp of a positive normal float
  return __uint_as_float(__float_as_uint(v) & 0x7F800000u) * 0x1p-23f;
}

__device__ __forceinline__ uint32_t wave_any(bool p) { return __ballot(p) != 0; }

__device__ __forceinline__ CodeCtx make_ctx(float ct, float mnew, float log2_15,
                                            float iscale = 0x1p-8f) {
  CodeCtx c;
  c.iscale = iscale;
  c.ct = ct;
  c.mnew = mnew;
  c.l2_15 = log2_15;
  // cq >= 2^-126: a score of -inf (a masked key of the last tile) then gives
  // t = -inf and y = 0 even when c_t = 0; for |I| < 2^14 the clamp moves t by
  // less than 2^-112, far inside the error bound below
  c.cq = fmaxf(ct * iscale, 0x1p-126f);
  c.m15n = log2_15 - mnew;
  // error of the fused argument against x + log2(15) for scores that can
  // round to a code in 1..15 (|x| < 8), in log2 units.  The fused product
  // I c_t is exact where m' = fl(max I c_t) is rounded, so the error grows
  // with |m'|; past 2^12 (logits of thousands of nats) the wave computes the
  // argument from x = fl(fl(I c_t) - m') <= 0 instead, whose only error is the
  // rounding of x + log2(15): y then never exceeds 15 (no overflow) and the
  // guard band stays narrow.
  float e = 0x1p-21f + ulp_pos(fabsf(mnew) + 8.0f);
  c.exact_arg = wave_any(e > 0x1p-12f);
  if (c.exact_arg) e = 0x1p-20f;
  // 15.5 * ln 2 < 10.75; v_exp_f32 error < 1 ulp; 12x and +4e-6 are margin.
  c.delta = 12.0f * e + 4e-6f;
  // c_t so small that c_t * iscale may be subnormal: never trust the fast path.
  if (ct != 0.0f && ct < 0x1p-100f) {
    c.delta = 1.0f;
  }
  return c;
}

// y ~ 15 * 2^x of NS scores (f = I / iscale exactly; a masked key arrives as
// -inf and gives y = 0), the argument taken as make_ctx decided for the wave.
// EA (exact argument) is that decision at compile time: the fp8 kernel takes
// it once per tile and runs one of two copies of its fast path.
template <int NS>
__device__ __forceinline__ void exp_scores_ea(const float (&f)[NS], const CodeCtx& cx,
                                              float (&y)[NS], bool ea) {
  if (!ea) {
#pragma unroll
    for (int r = 0; r < NS; ++r) y[r] = __builtin_amdgcn_exp2f(fmaf(f[r], cx.cq, cx.m15n));
  } else {
    const float ctc = fmaxf(cx.ct, 0x1p-126f);   // -inf * 0 would be NaN; see make_ctx
#pragma unroll
    for (int r = 0; r < NS; ++r)
      y[r] = __builtin_amdgcn_exp2f((f[r] * cx.iscale * ctc - cx.mnew) + cx.l2_15);
  }
}

template <int NS>
__device__ __forceinline__ void exp_scores(const float (&f)[NS], const CodeCtx& cx,
                                           float (&y)[NS]) {
  if (__builtin_expect(!cx.exact_arg, 1))
    exp_scores_ea<NS>(f, cx, y, false);
  else
    exp_scores_ea<NS>(f, cx, y, true);
}

// Exact P code of one score (float f = I / iscale exactly).
__device__ __forceinline__ int exact_code(float f, const CodeCtx& cx, const float* tau) {
  const float I = f * cx.iscale;   // exact (power of two)
  const float s = I * cx.ct;       // fl(I * c_t)
  const float x = s - cx.mnew;     // fl(s - m')
  int code = 0;
#pragma unroll
  for (int k = 0; k < 15; ++k) code += (x >= tau[k]) ? 1 : 0;
  return code;
}

// 16 scores of one lane (one 32-key subtile) -> 16 u4 codes packed in byte
// lanes (byte r = code of score r), and their unquantized 15*2^x added to lsum.
//
// fmax is the largest f of the group in this lane.  If in every lane of the
// wave even that score maps below 1/2 - delta, every code of the group is 0
// (exactly: exp2 and the fused argument are monotone, and the estimate is
// within delta of 15*2^x), so rounding, packing and the guard are skipped.
template <bool TAIL>
__device__ __forceinline__ v4i pcode16(const float (&f)[16], float fmax, const CodeCtx& cx,
                                       const float* tau, float& lsum, uint32_t valid) {
  float y[16], ym[1];
  exp_scores<16>(f, cx, y);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (TAIL) y[r] = ((valid >> r) & 1u) ? y[r] : 0.0f;
    lsum += y[r];
  }
  {
    const float fm[1] = {fmax};
    exp_scores<1>(fm, cx, ym);
  }
  const float ymax = ym[0];
  if (__builtin_expect(!wave_any(ymax >= 0.5f - cx.delta), 0)) return v4i{0, 0, 0, 0};
  float g = 1.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) g = fminf(g, fabsf(__builtin_amdgcn_fractf(y[r]) - 0.5f));
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * i], 0, 0u);
    v = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * i + 1], 1, v);
    v = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * i + 2], 2, v);
    pk[i] = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * i + 3], 3, v);
  }
  if (__builtin_expect(wave_any(g < cx.delta), 0)) {
    // rare: some score of the group sits within delta of a rounding boundary;
    // recompute the whole group exactly
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * i + j;
        int code = exact_code(f[r], cx, tau);
        if (TAIL && !((valid >> r) & 1u)) code = 0;
        v |= (uint32_t)code << (8 * j);
      }
      pk[i] = v;
    }
  }
  return v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
}

// P-code thresholds as the exact fix-up reads them: [0] = -inf, [k] = tau_k
// (k = 1..15), [16] = +inf.  Staged in LDS by every kernel that uses them.
constexpr int kTauTable = 17;

template <typename TauSrc>
__device__ __forceinline__ void stage_tau(const TauSrc& tau, float* t_lds) {
  for (int i = threadIdx.x; i < kTauTable; i += blockDim.x)
    t_lds[i] = i == 0 ? -INFINITY : (i == kTauTable - 1 ? INFINITY : tau[i - 1]);
}

// Sign bit of a float as 0/1: x >= t  <=>  sign(fl(x - t)) == 0 exactly
// (-0 and +0 included).
__device__ __forceinline__ int signbit01(float v) { return (int)(__float_as_uint(v) >> 31); }

// Fast P codes of one lane's 16 scores of a 32-key group (exact float I), as
// floats in rr (exact integers 0..15); lsum accumulates the unquantized
// 15*2^x (CS: the codes instead, the normalizer of the code-sum variant) and
// g the largest |y - rne(y)|.
//
// y = v_exp_f32(t), t = fma(I, c_t, log2(15) - m'), is within delta of
// 15*2^x, so rr = rne(y) is the exact code unless y lies within delta of a
// half-integer, i.e. unless g > 1/2 - delta; the caller checks g once for a
// whole tile and then fixes every code with exact_codes16.  Masked keys (last
// tile) arrive as I = -inf: t = -inf, y = 0, code 0.
template <bool CS = false, int EA = -1>
__device__ __forceinline__ void fast_codes16(const float (&f)[16], const CodeCtx& cx, float& lsum,
                                             float& g, float (&rr)[16]) {
  float y[16], d[16];
  if (EA < 0)
    exp_scores<16>(f, cx, y);
  else
    exp_scores_ea<16>(f, cx, y, EA != 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (!CS) lsum += y[r];
    rr[r] = __builtin_rintf(y[r]);
    d[r] = y[r] - rr[r];
    if (CS) lsum += rr[r];
  }
  // max |d| as a tree of v_max3 with |.| modifiers (depth 3) instead of one
  // chain of eight
  const float g0 = vmax3_abs(d[0], d[1], d[2]), g1 = vmax3_abs(d[3], d[4], d[5]);
  const float g2 = vmax3_abs(d[6], d[7], d[8]), g3 = vmax3_abs(d[9], d[10], d[11]);
  const float g4 = vmax3_abs(d[12], d[13], d[14]);
  g = vmax3(g, vmax3(g0, g1, g2), vmax3_abs(g3, g4, d[15]));
}

// Exact P codes from the fast ones.  |y - 15*2^x| < delta < 1/2, so the exact
// code is rr - 1, rr or rr + 1: it is rr - 1 iff x < tau_rr and rr + 1 iff
// x >= tau_{rr+1}, with x = fl(fl(I c_t) - m') and the staged table (tau_0 =
// -inf, tau_16 = +inf).  Masked keys give x = -inf (or NaN for c_t = 0), which
// no comparison accepts: code 0.
__device__ __forceinline__ void exact_codes16(const float (&f)[16], const CodeCtx& cx,
                                              const float* tau_lds, float (&rr)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int c0 = (int)rr[r];
    c0 = c0 < 0 ? 0 : (c0 > kTauTable - 2 ? kTauTable - 2 : c0);
    const float x = f[r] * cx.iscale * cx.ct - cx.mnew;   // fl(fl(I c_t) - m')
    const int code = c0 - (x < tau_lds[c0] ? 1 : 0) + (x >= tau_lds[c0 + 1] ? 1 : 0);
    rr[r] = (float)code;
  }
}

// The P codes of the fp8 kernel for 16 scores in one piece (fast codes, then
// the exact fix when the group's own guard trips): the self-test entry points
// run this on arbitrary scores.
template <bool CS = false, int EA = -1>
__device__ __forceinline__ void pcode16_f8(const float (&f)[16], const CodeCtx& cx,
                                           const float* tau_lds, float& lsum, float (&rr)[16]) {
  float g = 0.0f;
  fast_codes16<CS, EA>(f, cx, lsum, g, rr);
  // rare: laid out away from the common path
  if (__builtin_expect(wave_any(g > 0.5f - cx.delta), 0)) exact_codes16(f, cx, tau_lds, rr);
}

// The P^T operand of one 64-key chunk as FP6 E2M3: the 32 codes a lane holds
// for the chunk (a: its 16 keys of the first 32-key subtile, b: of the
// second), each as code/2.  v_cvt_scalef32_2xpk16_fp6_f32 packs src0[i] into
// 6-bit field 2i and src1[i] into field 2i + 1 (value / scale, scale 2), so
// field j < 16 holds a[j] and field 16 + j holds b[j].  The MFMA reads field j
// of a lane in half h as the key that byte 16h + j (j < 16) of the A operand's
// half 0 holds, and field 16 + j as byte 16h + j of half 1; the prologue's V^T
// order matches that.  The output must not share registers with the inputs
// (the conversion writes its result before it has read all of its sources),
// hence the early-clobber operand.
__device__ __forceinline__ v8i pack_p_fp6(const float (&a)[16], const float (&b)[16]) {
  v16f x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = a[2 * i];
    y[i] = a[2 * i + 1];
    x[8 + i] = b[2 * i];
    y[8 + i] = b[2 * i + 1];
  }
  v6i r;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, 2.0" : "=&v"(r) : "v"(x), "v"(y));
  return v8i{r[0], r[1], r[2], r[3], r[4], r[5], 0, 0};
}

// S^T tile MFMA: K x Q, both FP8 E4M3 (format 0) or both FP6 E2M3 (format 2,
// six dwords of each operand read); zero scales select the unscaled MFMA.
template <bool F6>
__device__ __forceinline__ v16f mfma_qk(const v8i& a, const v8i& b, const v16f& c) {
  if (F6) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, 0, 0, 0);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// V^T P^T MFMA: A (V^T) FP8 E4M3 or FP6 E2M3, B (P^T) FP6 E2M3.
template <bool F6>
__device__ __forceinline__ v16f mfma_pv(const v8i& a, const v8i& b, const v16f& c) {
  if (F6) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, 0, 0, 0);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 2, 0, 0, 0, 0);
}

template <int D, bool DBG>
struct Int4Kernel {
  static constexpr int KS = D / 32;        // k-steps of 32 channels for QK^T
  static constexpr int DB = D / 32;        // 32-channel blocks of O^T
  static constexpr int KStride = D + 16;   // K tile row in LDS (bytes)
  static constexpr int KB = D / 4;         // bytes of packed K (and of V^T) per thread per tile
  static constexpr int TPR = 256 / D;      // threads per packed V^T row

  // One key tile, part 1: S^T, running max, P codes.  TAIL: keys >= N exist
  // in this tile.
  template <bool TAIL>
  __device__ __forceinline__ static void scores(const Int4Args& a, const Int4Debug& dbg, int bh,
                                                int t, const uint8_t* sk, const v4i (&qf)[KS],
                                                float qs, float& m, float& l, v16f (&O)[DB],
                                                v4i (&P)[4]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const size_t sidx = (size_t)bh * a.NB + t;

    v16i S[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      S[sub] = v16i{0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v4i kf = *(const v4i*)(sk + (32 * sub + col) * KStride + 32 * ks + 16 * hh);
        S[sub] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[ks], S[sub], 0, 0, 0);
      }
    }

    uint32_t valid[4] = {0xffffu, 0xffffu, 0xffffu, 0xffffu};
    if (TAIL) {
      const int nv = a.N - t * kBlock;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        uint32_t vm = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key < nv) vm |= 1u << r;
          else S[sub][r] = INT32_MIN;
        }
        valid[sub] = vm;
      }
    }

    int smx[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      smx[sub] = S[sub][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) smx[sub] = max(smx[sub], S[sub][r]);
    }
    int mx = max(max(smx[0], smx[1]), max(smx[2], smx[3]));
    mx = max(mx, other_half(mx));

    const float ct = qs * a.k_scale[sidx];
    const float smax = (float)(mx >> 8) * ct;
    const float mnew = fmaxf(m, smax);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    if (wave_any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    m = mnew;
    const CodeCtx cx = make_ctx(ct, mnew, a.log2_15);

    // the tile's terms are summed on their own first: adding ~10^4 terms per
    // lane straight into the running l would drop the ones below half an ulp
    float ls = 0.0f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      float f[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) f[r] = (float)S[sub][r];
      P[sub] = pcode16<TAIL>(f, (float)smx[sub], cx, a.tau, ls, valid[sub]);
    }
    l = fmaf(l, alpha, ls);

    if (DBG) {
      const int q = 32 * w + col;
      const size_t npad = (size_t)a.NB * kBlock;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const size_t key = (size_t)t * kBlock + 32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3);
          dbg.s_int[q * npad + key] = S[sub][r] >> 8;
          dbg.p_code[q * npad + key] = (uint8_t)((uint32_t)P[sub][r >> 2] >> (8 * (r & 3)));
        }
    }

  }

  // One key tile, part 2: O^T = alpha O^T + (v_scale/16) V^T P^T.
  __device__ __forceinline__ static void pv(const Int4Args& a, const Int4Debug& dbg, int bh, int t,
                                            const uint8_t* sv, const v4i (&P)[4], v16f (&O)[DB]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const float sv16 = a.v_scale[(size_t)bh * a.NB + t] * 0.0625f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      v16i pv = v16i{0};
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const v4i vf = *(const v4i*)(sv + (32 * db + col) * kVStride + 32 * sub + 16 * hh);
        pv = __builtin_amdgcn_mfma_i32_32x32x32_i8(vf, P[sub], pv, 0, 0, 0);
      }
      if (DBG) {
        const int q = 32 * w + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
          dbg.pv_int[((size_t)t * kBlock + q) * D + d] = pv[r] >> 4;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) O[db][r] = fmaf((float)pv[r], sv16, O[db][r]);
    }
  }

  __device__ static void run(const Int4Args& a, const Int4Debug& dbg) {
    __shared__ __align__(16) uint8_t sk[2][kBlock * KStride];
    __shared__ __align__(16) uint8_t sv[2][D * kVStride];
    const int qb = DBG ? dbg.q_block : blockIdx.x;
    const int bh = DBG ? dbg.bh : blockIdx.y;
    if (!DBG && !a.run.test(bh)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int NB = a.NB;
    const size_t rows0 = (size_t)bh * NB * kBlock;   // first packed row of this head

    v4i qf[KS];
    {
      const uint8_t* qrow = a.q4 + (rows0 + (size_t)qb * kBlock + 32 * w + col) * (D / 2);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint2 p = *(const uint2*)(qrow + 16 * ks + 8 * hh);
        qf[ks] = v4i{(int)unpack_lo(p.x), (int)unpack_hi(p.x), (int)unpack_lo(p.y),
                     (int)unpack_hi(p.y)};
      }
    }
    const float qs = a.q_scale_l2[(size_t)bh * NB + qb];

    uint4 kreg[KB / 16], vreg[KB / 16];
    auto gload = [&](int t) {
      const uint8_t* ks = a.k4 + (rows0 + (size_t)t * kBlock + (tid >> 1)) * (D / 2) + (tid & 1) * KB;
      const uint8_t* vs = a.v4 + (((size_t)bh * NB + t) * D + tid / TPR) * 64 + (tid % TPR) * KB;
#pragma unroll
      for (int i = 0; i < KB / 16; ++i) {
        kreg[i] = *(const uint4*)(ks + 16 * i);
        vreg[i] = *(const uint4*)(vs + 16 * i);
      }
    };
    auto lstore = [&](int buf) {
      uint8_t* kd = sk[buf] + (tid >> 1) * KStride + (tid & 1) * (D / 2);
      uint8_t* vd = sv[buf] + (tid / TPR) * kVStride + (tid % TPR) * (D / 2);
#pragma unroll
      for (int i = 0; i < KB / 16; ++i) {
        const uint4 p = kreg[i];
        *(uint4*)(kd + 32 * i) = uint4{unpack_lo(p.x), unpack_hi(p.x), unpack_lo(p.y), unpack_hi(p.y)};
        *(uint4*)(kd + 32 * i + 16) = uint4{unpack_lo(p.z), unpack_hi(p.z), unpack_lo(p.w), unpack_hi(p.w)};
        // V^T: a packed 16-byte chunk is one 32-key subtile (groups g = 0..3 of 8
        // keys).  Dword slot s of the subtile row receives keys
        // 8(s%4) + 4(s/4) .. +3, which is the key order of the P^T operand
        // taken straight from the S^T accumulator layout.
        const uint4 q = vreg[i];
        *(uint4*)(vd + 32 * i) = uint4{unpack_lo(q.x), unpack_lo(q.y), unpack_lo(q.z), unpack_lo(q.w)};
        *(uint4*)(vd + 32 * i + 16) = uint4{unpack_hi(q.x), unpack_hi(q.y), unpack_hi(q.z), unpack_hi(q.w)};
      }
    };

    float m = -INFINITY, l = 0.0f;
    v16f O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = v16f{0.0f};

    const int NT = NB;
    gload(0);
    lstore(0);
    __syncthreads();
    // every tile but the last is full; the last one is peeled off so that the
    // loop body has a single path (no accumulator copies between variants)
#pragma unroll 1
    for (int t = 0; t < NT - 1; ++t) {
      const int buf = t & 1;
      v4i P[4];
      scores<false>(a, dbg, bh, t, sk[buf], qf, qs, m, l, O, P);
      // the next tile's global loads overlap the P.V products; issuing them
      // here keeps their registers off the score phase's peak
      gload(t + 1);
      pv(a, dbg, bh, t, sv[buf], P, O);
      lstore(buf ^ 1);
      __syncthreads();
    }
    {
      const int t = NT - 1, buf = t & 1;
      v4i P[4];
      if ((a.N % kBlock) != 0)
        scores<true>(a, dbg, bh, t, sk[buf], qf, qs, m, l, O, P);
      else
        scores<false>(a, dbg, bh, t, sk[buf], qf, qs, m, l, O, P);
      pv(a, dbg, bh, t, sv[buf], P, O);
    }

    l += other_half(l);
    const int query = qb * kBlock + 32 * w + col;
    if (DBG && hh == 0) {
      dbg.m_final[32 * w + col] = m;
      dbg.l_final[32 * w + col] = l * (1.0f / 15.0f);
    }
    if (query < a.N) {
      const float il = 1.0f / l;
      uint16_t* orow = a.o + a.os.head_offset(bh, a.H) + (int64_t)query * a.os.token;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * hh;
          uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * g] * il)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * g + 1] * il)) << 16);
          uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * g + 2] * il)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * g + 3] * il)) << 16);
          *(uint2*)(orow + d0) = uint2{w0, w1};
        }
    }
  }
};

template <int D, bool DBG>
__global__ __launch_bounds__(kThreads, 2) void k_int4_attn(Int4Args a, Int4Debug dbg) {
  Int4Kernel<D, DBG>::run(a, dbg);
}

hipError_t launch_int4(int D, int BH, const Int4Args& a, const Int4Debug* dbg, hipStream_t st) {
  Int4Debug none{};
  if (dbg == nullptr) {
    dim3 grid(a.NB, BH);
    if (D == 128)
      hipLaunchKernelGGL((k_int4_attn<128, false>), grid, dim3(kThreads), 0, st, a, none);
    else
      hipLaunchKernelGGL((k_int4_attn<64, false>), grid, dim3(kThreads), 0, st, a, none);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((k_int4_attn<128, true>), dim3(1), dim3(kThreads), 0, st, a, *dbg);
    else
      hipLaunchKernelGGL((k_int4_attn<64, true>), dim3(1), dim3(kThreads), 0, st, a, *dbg);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- fp8 kernel
//
// The INT4 attention on the FP8-lane layout (codes as E4M3 bytes) or on the
// FP6 layout (codes as E2M3 fields: the integers -7..7 are exact there too):
//   S^T  = K_t Q^T on v_mfma_f32_32x32x64_f8f6f4: the fp32 result is I exactly
//          (integer products and partial sums below 2^24)
//   O^T  accumulates V_t^T (P/2)^T straight into fp32 on the same MFMA (V^T
//        FP8 or FP6, P as FP6 E2M3 code/2), kept in units of the current V
//        block scale u: O <- beta O + V^T (P/2)^T with beta = 2^(m-m') u_prev / u.
//        The final O is 2 O u / l.
// With both operands FP6 the MFMA runs at twice the FP8 rate.  The FP6 layout
// keeps the FP8 layout's byte positions: each 32-code operand group is 24
// bytes of fields and 8 bytes of padding, so the tiles, their swizzle and the
// operand offsets are the same, and an operand read is 24 bytes, not 32.
// No unpacking (the prologue stores operand-ready bytes) and no int->float
// conversions; per score the VALU work is the fused argument, exp2, the l
// sum, rndne and the guard, plus 1/32 of a packing instruction (32 codes to
// FP6 in one v_cvt_scalef32_2xpk16_fp6_f32: ~2.1 SIMD clocks per code
// against ~4.8 for the two-at-a-time FP8 conversion).
// One work-group = 4 waves = one 128-query block of one head, 32 queries per
// wave; two work-groups per CU, so that on each SIMD one wave's softmax (VALU)
// overlaps the other's MFMAs, which run at raised wave priority.  Per tile:
// S, softmax, then the K/V tiles of t+1 are requested straight into the other
// LDS buffers (global_load_lds) while P.V of tile t runs; one barrier per tile.
template <int D, bool DBG, bool CS, bool F6>
struct Int4F8Kernel {
  static constexpr int KS = D / 64;        // k-steps of 64 channels for QK^T
  static constexpr int DB = D / 32;        // 32-channel blocks of O^T
  static constexpr int NTHR = 256;
  // K tiles ([128 keys][D]) and V^T tiles ([D][128 keys]) sit unpadded in LDS,
  // filled by global_load_lds_dwordx4 (lane L of a wave writes bytes 16L..16L+15
  // of the wave's 1 KiB window); their 16-byte chunks are XOR-swizzled per row
  // so that the MFMA operand reads of 8 consecutive rows hit 8 different chunk
  // columns (all 32 banks).
  static constexpr int KCPR = D / 16;                  // chunks per K row
  static constexpr int KROWS128 = 128 / D;             // K rows per 128 bytes
  static constexpr int KCHUNKS = kBlock * D / 16;      // chunks per tile (K or V^T)
  static constexpr int LOADS = KCHUNKS / NTHR;         // load instructions per thread per tile
  static constexpr int NW = NTHR / 64;                 // waves
  static_assert(KCHUNKS % NTHR == 0, "whole waves per tile");

  __device__ __forceinline__ static int kswz(int row) { return (row / (2 * KROWS128)) & (KCPR - 1); }
  __device__ __forceinline__ static int vswz(int row) { return (row >> 1) & 7; }

  __device__ __forceinline__ static v8i ld32(const uint8_t* p) {
    const uint4 a = *(const uint4*)p;
    if (F6) {
      const uint2 b = *(const uint2*)(p + 16);
      // dwords 6 and 7 are not read by an FP6 operand: left undefined (no moves)
      const int u = __builtin_nondeterministic_value(0);
      return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, u, u};
    }
    const uint4 b = *(const uint4*)(p + 16);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
  // 32 bytes of a swizzled row: logical chunks c0, c0 + 1
  __device__ __forceinline__ static v8i ld32s(const uint8_t* row, int c0, int key) {
    const uint4 a = *(const uint4*)(row + 16 * (c0 ^ key));
    const uint4 b = *(const uint4*)(row + 16 * ((c0 + 1) ^ key));
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
  // The same for the operand reads of the MFMA loops: logical chunk
  // 4k + 2hh + j of row r (j = 0, 1) sits at byte 16 ((2hh ^ key(r)) ^ (4k + j))
  // of the row (the three index parts use disjoint bits), so one per-lane
  // offset x = row * width + 16 (2hh ^ key) serves every k and j by an XOR.
  // x is made opaque once per tile so that the four XORed offsets are
  // recomputed (3 VALU) instead of being held in registers across the loop.
  __device__ __forceinline__ static v8i ld32x(const uint8_t* tile, uint32_t x, int k) {
    const uint4 a = *(const uint4*)(tile + (x ^ (64u * k)));
    if (F6) {
      // a whole 16-byte read (fields 16..23 and the pad): 8-byte reads get
      // paired across subtiles by the compiler and then moved into place
      v4i b = *(const v4i*)(tile + (x ^ (64u * k + 16u)));
      asm volatile("" : "+v"(b));
      return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, b[0], b[1], b[2], b[3]};
    }
    const uint4 b = *(const uint4*)(tile + (x ^ (64u * k + 16u)));
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }

  // S^T = K_t Q^T
  __device__ __forceinline__ static void qk(const uint8_t* sk, const v8i (&qf)[KS], v16f (&S)[4]) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, hh = lane >> 5;
    uint32_t x = col * D + 16 * ((2 * hh) ^ kswz(col));
    asm volatile("" : "+v"(x));
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      S[sub] = v16f{0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        S[sub] = mfma_qk<F6>(ld32x(sk + 32 * sub * D, x, ks), qf[ks], S[sub]);
    }
  }

  // O^T += V_t^T (P/2)^T  (P as FP6 code/2: the product is PV/2 exactly)
  __device__ __forceinline__ static void pv(const Int4Debug& dbg, int t, const uint8_t* sv,
                                            const v8i (&P)[2], v16f (&O)[DB]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 31, hh = lane >> 5;
    uint32_t xv = col * kBlock + 16 * ((2 * hh) ^ vswz(col));
    if (!DBG) asm volatile("" : "+v"(xv));
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 32 * db + col;
      if (DBG) {
        v16f pvt = v16f{0.0f};
#pragma unroll
        for (int c = 0; c < 2; ++c)
          pvt = mfma_pv<F6>(ld32s(sv + row * kBlock, 4 * c + 2 * hh, vswz(row)), P[c], pvt);
        const int q = 32 * w + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
          dbg.pv_int[((size_t)t * kBlock + q) * D + d] = (int32_t)(2.0f * pvt[r]);
          O[db][r] += pvt[r];
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c)
          O[db] = mfma_pv<F6>(ld32x(sv + 32 * db * kBlock, xv, c), P[c], O[db]);
      }
    }
  }

  // Keys >= nv of the tile (last tile only) get S = -inf: they then take no
  // part in the max, and give y = 0 and code 0.
  __device__ __forceinline__ static void mask_tail(v16f (&S)[4], int nv) {
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= nv) S[sub][r] = -INFINITY;
      }
  }

  // Softmax of key tile t (nv valid keys): running max, rescale of O, P codes,
  // row sum.
  __device__ __forceinline__ static void softmax(const Int4Args& a, const Int4Debug& dbg,
                                                 const float* tau_lds, const uint8_t* sk,
                                                 const v8i (&qf)[KS], int bh, int t, int nv,
                                                 v16f (&S)[4], float qs, float& m, float& l,
                                                 float& u, v16f (&O)[DB], v8i (&P)[2]) {
    const int lane = threadIdx.x & 63, wl = threadIdx.x >> 6;
    const int hh = lane >> 5, col = lane & 31;
    const size_t sidx = (size_t)bh * a.NB + t;

    // row max as plain v_max3 chains: the scores are exact integers or -inf,
    // never NaN, so the quieting that fmaxf needs on MFMA results is dropped
    // (trees: depth 3 per subtile instead of chains of seven)
    float smx[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const v16f& x = S[sub];
      const float a0 = vmax3(x[0], x[1], x[2]), a1 = vmax3(x[3], x[4], x[5]);
      const float a2 = vmax3(x[6], x[7], x[8]), a3 = vmax3(x[9], x[10], x[11]);
      const float a4 = vmax3(x[12], x[13], x[14]);
      smx[sub] = vmax3(vmax3(a0, a1, a2), a3, vmax3(a4, x[15], x[15]));
    }
    float mx = vmax2(vmax3(smx[0], smx[1], smx[2]), smx[3]);
    mx = vmax2(mx, other_half(mx));

    // the block scales are read through the scalar unit (uniform address):
    // as vector loads they would sit behind the next tile's loads in vmcnt order
    typedef const __attribute__((address_space(4))) float* cfloat_ptr;
    const float ct = qs * ((cfloat_ptr)a.k_scale)[sidx];
    const float mnew = vmax2(m, mx * ct);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    // O is kept in units of the current tile's V scale; a rescale error of an
    // ulp is far below the fp16 output rounding
    const float sv = ((cfloat_ptr)a.v_scale)[sidx];
    const float unew = sv > 0.0f ? sv : u;
    const float beta = alpha * (u * __builtin_amdgcn_rcpf(unew));
    u = unew;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[db][r] *= beta;
    const CodeCtx cx = make_ctx(ct, mnew, a.log2_15, 1.0f);

    // P codes per 32-key subtile, each with its own (rarely taken) exact fix;
    // the exponent-argument form is decided once per tile.  One partial sum
    // per subtile: four independent add chains (-0 + y == y for every y: no
    // add of a zero start)
    float lsp[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
    float rr[4][16];
    auto codes = [&](auto ea) {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        float f[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) f[r] = S[sub][r];
        pcode16_f8<CS, decltype(ea)::value>(f, cx, tau_lds, lsp[sub], rr[sub]);
      }
    };
    if (__builtin_expect(!cx.exact_arg, 1))
      codes(std::integral_constant<int, 0>{});
    else
      codes(std::integral_constant<int, 1>{});
    // 64-key chunk c = subtiles 2c and 2c+1
    P[0] = pack_p_fp6(rr[0], rr[1]);
    P[1] = pack_p_fp6(rr[2], rr[3]);
    l = fmaf(l, alpha, (lsp[0] + lsp[1]) + (lsp[2] + lsp[3]));

    if (DBG) {
      const int q = 32 * wl + col;
      const size_t npad = (size_t)a.NB * kBlock;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kt = 32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3);
          const size_t key = (size_t)t * kBlock + kt;
          dbg.s_int[q * npad + key] = kt >= nv ? INT32_MIN : (int32_t)S[sub][r];
          dbg.p_code[q * npad + key] = (uint8_t)rr[sub][r];
        }
    }
  }

  __device__ static void run(const Int4Args& a, const Int4Debug& dbg) {
    __shared__ __align__(16) uint8_t sk[2][kBlock * D];
    __shared__ __align__(16) uint8_t sv[2][D * kBlock];
    __shared__ float tau_lds[kTauTable];
    const int qb = DBG ? dbg.q_block : blockIdx.x;
    const int bh = DBG ? dbg.bh : blockIdx.y;
    if (!DBG && !a.run.test(bh)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int NB = a.NB, NT = NB;
    const size_t rows0 = (size_t)bh * NB * kBlock;
    stage_tau(a.tau, tau_lds);

    v8i qf[KS];
    {
      const uint8_t* qrow = a.q4 + (rows0 + (size_t)qb * kBlock + 32 * w + col) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = ld32(qrow + 64 * ks + 32 * hh);
    }
    const float qs = a.q_scale_l2[(size_t)bh * NB + qb];

    // tile loads straight into LDS (no registers): wave w, instruction i fills
    // chunks (NW i + w) * 64 + lane of the tile.  The per-lane byte offsets
    // within a tile are fixed; only the tile base (uniform) moves.
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int wu = __builtin_amdgcn_readfirstlane(w);   // wave index in an SGPR (LDS window base)
    // Instruction i of a wave fills rows 32i (D = 128; 64i for D = 64) further
    // down than instruction 0, and the swizzle keys repeat with that period,
    // so its per-lane offset is instruction 0's plus 4096 i: the uniform part
    // goes to the scalar base, and one offset register per tensor remains.
    static_assert(NW * 64 * 16 == 4096, "4 KiB per load instruction of the work-group");
    uint32_t koff0, voff0;
    {
      const int pc = w * 64 + lane;                        // physical chunk of instruction 0
      const int krow = pc / KCPR, vrow = pc / 8;
      koff0 = krow * D + 16 * ((pc % KCPR) ^ kswz(krow));
      voff0 = vrow * kBlock + 16 * ((pc % 8) ^ vswz(vrow));
    }
    auto gload = [&](int t, int buf) {
      const uint8_t* kb = a.k4 + (rows0 + (size_t)t * kBlock) * D;
      const uint8_t* vb = a.v4 + ((size_t)bh * NB + t) * D * kBlock;
      // opaque per tile: keeps the loop from turning base + offset into
      // per-lane 64-bit pointers held in registers
      uint32_t ko = koff0, vo = voff0;
      asm volatile("" : "+v"(ko), "+v"(vo));
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        // uniform base in an SGPR pair + 32-bit lane offset: the saddr form
        const uint8_t* kbi = kb + 4096 * i;
        const uint8_t* vbi = vb + 4096 * i;
        asm volatile("" : "+s"(kbi), "+s"(vbi));
        __builtin_amdgcn_global_load_lds((const void*)(kbi + ko),
                                         (lds_ptr)(sk[buf] + (NW * i + wu) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vbi + vo),
                                         (lds_ptr)(sv[buf] + (NW * i + wu) * 1024), 16, 0, 0);
      }
    };

    float m = -INFINITY, l = 0.0f, u = 1.0f;
    v16f O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = v16f{0.0f};
    const int nv_last = a.N - (NT - 1) * kBlock;   // valid keys of the last tile

    gload(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll 1
    for (int t = 0; t < NT; ++t) {
      const int buf = t & 1;
      v16f S[4];
      v8i P[2];
      __builtin_amdgcn_s_setprio(1);
      qk(sk[buf], qf, S);
      __builtin_amdgcn_s_setprio(0);
      int nv = kBlock;
      if (__builtin_expect(t == NT - 1 && nv_last < kBlock, 0)) {
        // opaque: nv_last is loop-invariant, and the 64 comparisons would be
        // hoisted out of the loop and kept live (as SGPR masks) throughout it
        nv = nv_last;
        asm volatile("" : "+v"(nv));
        mask_tail(S, nv);
      }
      softmax(a, dbg, tau_lds, sk[buf], qf, bh, t, nv, S, qs, m, l, u, O, P);
      // tile t+1 -> the other buffers, last read in tile t-1 (before the barrier)
      if (t + 1 < NT) gload(t + 1, buf ^ 1);
      __builtin_amdgcn_s_setprio(1);
      pv(dbg, t, sv[buf], P, O);
      __builtin_amdgcn_s_setprio(0);
      // this thread's tile loads have landed in LDS before anyone passes the barrier
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    l += other_half(l);
    const int query = qb * kBlock + 32 * w + col;
    if (DBG && hh == 0) {
      dbg.m_final[32 * w + col] = m;
      dbg.l_final[32 * w + col] = l * (1.0f / 15.0f);
    }
    if (query < a.N) {
      const float il = 2.0f * u / l;   // O accumulated PV/2
      uint16_t* orow = a.o + a.os.head_offset(bh, a.H) + (int64_t)query * a.os.token;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = 32 * db + 8 * gq + 4 * hh;
          uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * gq] * il)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * gq + 1] * il)) << 16);
          uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * gq + 2] * il)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[db][4 * gq + 3] * il)) << 16);
          *(uint2*)(orow + d0) = uint2{w0, w1};
        }
    }
  }
};

template <int D, bool DBG, bool CS, bool F6>
__global__ __launch_bounds__(256, 2) void k_int4_attn_f8(Int4Args a, Int4Debug dbg) {
  Int4F8Kernel<D, DBG, CS, F6>::run(a, dbg);
}

template <int D, bool CS, bool F6>
static void launch_int4_f8_t(int BH, const Int4Args& a, const Int4Debug* dbg, hipStream_t st) {
  if (dbg == nullptr) {
    Int4Debug none{};
    hipLaunchKernelGGL((k_int4_attn_f8<D, false, CS, F6>), dim3(a.NB, BH), dim3(256), 0, st, a,
                       none);
  } else {
    hipLaunchKernelGGL((k_int4_attn_f8<D, true, CS, F6>), dim3(1), dim3(256), 0, st, a, *dbg);
  }
}

template <int D>
static void launch_int4_f8_d(int BH, const Int4Args& a, const Int4Debug* dbg, hipStream_t st) {
  if (a.f6)
    a.code_sum ? launch_int4_f8_t<D, true, true>(BH, a, dbg, st)
               : launch_int4_f8_t<D, false, true>(BH, a, dbg, st);
  else
    a.code_sum ? launch_int4_f8_t<D, true, false>(BH, a, dbg, st)
               : launch_int4_f8_t<D, false, false>(BH, a, dbg, st);
}

hipError_t launch_int4_f8(int D, int BH, const Int4Args& a, const Int4Debug* dbg, hipStream_t st) {
  if (D == 128)
    launch_int4_f8_d<128>(BH, a, dbg, st);
  else
    launch_int4_f8_d<64>(BH, a, dbg, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- self-tests

struct SweepArgs {
  float tau[15];
  float log2_15;
  uint32_t mag_lo, count, max_trans;
  uint32_t *trans, *n_trans;
};

// The code path of the packed (i8) or the fp8 kernel over 16 scores given as
// exact I (float), as u8 codes in byte lanes.
template <bool F8>
__device__ __forceinline__ v4i codes_of(const float (&I)[16], float c, float m, const SweepArgs& a,
                                        const float* tau, const float* tau_lds) {
  float f[16], fm = -INFINITY, ls = 0.0f;
  const float sc = F8 ? 1.0f : 256.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    f[r] = I[r] * sc;
    fm = fmaxf(fm, f[r]);
  }
  if (F8) {
    const CodeCtx cx = make_ctx(c, m, a.log2_15, 1.0f);
    float rr[16], lsum = 0.0f;
    pcode16_f8(f, cx, tau_lds, lsum, rr);   // codes as exact floats
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = __builtin_amdgcn_cvt_pk_u8_f32(rr[4 * i], 0, 0u);
      v = __builtin_amdgcn_cvt_pk_u8_f32(rr[4 * i + 1], 1, v);
      v = __builtin_amdgcn_cvt_pk_u8_f32(rr[4 * i + 2], 2, v);
      pk[i] = __builtin_amdgcn_cvt_pk_u8_f32(rr[4 * i + 3], 3, v);
    }
    return v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
  } else {
    const CodeCtx cx = make_ctx(c, m, a.log2_15);
    return pcode16<false>(f, fm, cx, tau, ls, 0xffffu);
  }
}

// Each lane evaluates 16 consecutive magnitudes (x = -magnitude, c = 1, m = 0)
// and the 16 magnitudes one below, then reports every change of code.
template <bool F8>
__global__ __launch_bounds__(256) void k_pcode_sweep(SweepArgs a) {
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  const uint32_t b0 = a.mag_lo + 16u * idx;
  float I[16], Ip[16];
  uint32_t live = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t b = b0 + r;
    const bool in = (16u * idx + r) < a.count;
    live |= (in ? 1u : 0u) << r;
    const uint32_t bp = b == 0 ? 0u : b - 1u;
    I[r] = -__uint_as_float(in ? b : 0u);
    Ip[r] = -__uint_as_float(in ? bp : 0u);
  }
  __shared__ float tau_lds[kTauTable];
  stage_tau(a.tau, tau_lds);
  __syncthreads();
  const v4i c = codes_of<F8>(I, 1.0f, 0.0f, a, a.tau, tau_lds);
  const v4i cp = codes_of<F8>(Ip, 1.0f, 0.0f, a, a.tau, tau_lds);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t cc = ((uint32_t)c[r >> 2] >> (8 * (r & 3))) & 0xffu;
    const uint32_t pc = ((uint32_t)cp[r >> 2] >> (8 * (r & 3))) & 0xffu;
    if (((live >> r) & 1u) && cc != pc) {
      const uint32_t i = atomicAdd(a.n_trans, 1u);
      if (i < a.max_trans) {
        a.trans[3 * i] = b0 + r;
        a.trans[3 * i + 1] = pc;
        a.trans[3 * i + 2] = cc;
      }
    }
  }
}

hipError_t launch_pcode_sweep(bool f8, uint32_t mag_lo, uint32_t count, const float tau[15],
                              float log2_15, uint32_t* transitions, uint32_t max_transitions,
                              uint32_t* n_trans, hipStream_t st) {
  SweepArgs a;
  for (int k = 0; k < 15; ++k) a.tau[k] = tau[k];
  a.log2_15 = log2_15;
  a.mag_lo = mag_lo;
  a.count = count;
  a.max_trans = max_transitions;
  a.trans = transitions;
  a.n_trans = n_trans;
  const uint32_t lanes = (count + 15u) / 16u;
  const uint32_t blocks = (lanes + 255u) / 256u;
  if (f8)
    hipLaunchKernelGGL(k_pcode_sweep<true>, dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_pcode_sweep<false>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

struct EvalArgs {
  SweepArgs s;
  float c, m;
  const int32_t* I;
  uint8_t* codes;
};

template <bool F8>
__global__ __launch_bounds__(256) void k_pcode_eval(EvalArgs a) {
  const size_t base = ((size_t)blockIdx.x * 256u + threadIdx.x) * 16u;
  float I[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) I[r] = (float)a.I[base + r];
  __shared__ float tau_lds[kTauTable];
  stage_tau(a.s.tau, tau_lds);
  __syncthreads();
  *(v4i*)(a.codes + base) = codes_of<F8>(I, a.c, a.m, a.s, a.s.tau, tau_lds);
}

hipError_t launch_pcode_eval(bool f8, const int32_t* I, uint32_t n, float c, float m,
                             const float tau[15], float log2_15, uint8_t* codes, hipStream_t st) {
  EvalArgs a;
  for (int k = 0; k < 15; ++k) a.s.tau[k] = tau[k];
  a.s.log2_15 = log2_15;
  a.c = c;
  a.m = m;
  a.I = I;
  a.codes = codes;
  if (f8)
    hipLaunchKernelGGL(k_pcode_eval<true>, dim3(n / 4096u), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_pcode_eval<false>, dim3(n / 4096u), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace rotattn

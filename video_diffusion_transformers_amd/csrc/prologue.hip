// K1: the RotateAttention prologue on gfx950.
//
// RotateAttention (page title "RotateAttention: RoPE-Aware Rotation and Range
// Rectification for INT4 Quantized Attention in Video Generation", Abstract):
// Q and K of a DiT video model carry 3D RoPE; their outliers sit in channels
// laid out by RoPE's partitions, so an orthogonal rotation applied inside each
// RoPE partition after RoPE (which leaves QK^T unchanged) spreads them before
// symmetric INT4 quantization.  Heads routed to the FP16 fallback only get
// RoPE'd fp16 Q/K.
//
// One work-group per (128-token block, head); 256 threads = 4 waves, one per
// SIMD, so that two work-groups share a CU whatever their wave placement.
// Arithmetic (bit-exact by construction; this file is built with
// -ffp-contract=off):
//   RoPE   y0 = fl(fl(x0*c) - fl(x1*s)), y1 = fl(fl(x0*s) + fl(x1*c))   fp32
//   rotate z_r = fl32(sum_k R[r][k]*y_k) in fp64, k ascending (the fp32 x fp32
//          products are exact in fp64), one rounding to fp32
//   INT4   per block: amax over the 128 tokens x D channels, inv = fl(7/amax),
//          scale = fl(amax/7), code = clamp(rne(fl(z*inv)), -7, 7)
// The rotation of a partition is a [128 tokens x d_a] x [d_a x d_a] product and
// runs on v_mfma_f64_16x16x4_f64, which accumulates D = C + a0 b0 + a1 b1 +
// a2 b2 + a3 b3 as a chain of fused multiply-adds in ascending k (checked
// bit for bit on the device against that chain), so 16x16x4 steps chained over
// k reproduce the sequential fp64 sum exactly.  Wave w owns tokens
// 32w..32w+31 in every partition: R_a^T is read (from cache) into registers
// as B fragments partition by partition, and the A fragments are RoPE'd on
// the fly from the staged fp16 rows.
#include "rotattn_internal.h"

namespace rotattn {

constexpr int kThreads = 256;
constexpr int kCodeStride = 132;   // bytes per row of the int8 code buffers (33 dwords: no bank conflicts)

// Thread index within the 256 threads that run one prologue unit (a 128-token
// block of one tensor of one head): the whole work-group in the kernels with
// 256 threads, one half of it in the 512-thread QKV projection, whose halves
// run two units side by side (same code path, so the same barriers).
__device__ __forceinline__ int ltid() { return threadIdx.x & (kThreads - 1); }

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// RoPE of this lane's token over one partition of width DA at channel offset
// off: y[0..DA) in fp32.  xrow is the token's fp16 row staged in LDS (one
// dword per channel pair).
template <int DA>
__device__ __forceinline__ void rope_part(const uint32_t* xrow, const float* cos_a,
                                          const float* sin_a, int pos, int off, float (&y)[DA]) {
#pragma unroll
  for (int j = 0; j < DA / 2; ++j) {
    const uint32_t pr = xrow[off / 2 + j];
    const float x0 = h2f((uint16_t)(pr & 0xffffu));
    const float x1 = h2f((uint16_t)(pr >> 16));
    const float c = cos_a[pos * (DA / 2) + j];
    const float s = sin_a[pos * (DA / 2) + j];
    y[2 * j] = x0 * c - x1 * s;
    y[2 * j + 1] = x0 * s + x1 * c;
  }
}

__global__ void k_rot_to_f64(const float* rt, const float* rh, const float* rw, int dt, int dh,
                             double* out) {
  const int total = dt * dt + 2 * dh * dh;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    int j = i, w_ = dt;
    const float* src = rt;
    if (i >= dt * dt) {
      j = i - dt * dt;
      const int p = j >= dh * dh;
      j -= p * dh * dh;
      w_ = dh;
      src = p ? rw : rh;
    }
    const int k = j / w_, r = j % w_;              // stored [k][r] from R[r][k]
    out[i] = (double)src[r * w_ + k];
  }
  // the prologue's B fragments of R_a^T, fp32, lane-major (see load_rot_frags)
  float* frag = (float*)((uint8_t*)out + kRotFragOffset);
  const int nfrag = 3 * 64 * kRotFragStride;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nfrag; i += gridDim.x * blockDim.x) {
    const int part = i / (64 * kRotFragStride), rem = i % (64 * kRotFragStride);
    const int l = rem / kRotFragStride, e = rem % kRotFragStride;
    const int w_ = part == 0 ? dt : dh;
    const float* src = part == 0 ? rt : (part == 1 ? rh : rw);
    const int JB = (w_ + 15) / 16, KS = (w_ + 3) / 4;
    const int ks = e / JB, jb = e % JB;
    const int k = 4 * ks + l / 16, j = 16 * jb + l % 16;
    frag[i] = (ks < KS && k < w_ && j < w_) ? src[j * w_ + k] : 0.0f;
  }
}

hipError_t launch_rot_to_f64(const float* rt, const float* rh, const float* rw, int dt, int dh,
                             double* out, hipStream_t st) {
  hipLaunchKernelGGL(k_rot_to_f64, dim3(16), dim3(256), 0, st, rt, rh, rw, dt, dh, out);
  return hipGetLastError();
}

// The three axes' RoPE tables as (cos, sin) pairs: one 8-byte load per
// channel pair in the prologue instead of two.
__global__ void k_rope_pairs(rotattn_rope_rot rr, int np_t, int np_h, int np_w, float* out) {
  const int total = np_t + np_h + np_w;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const float *c = rr.cos_t, *s = rr.sin_t;
    int j = i;
    if (j >= np_t) {
      j -= np_t;
      c = rr.cos_h;
      s = rr.sin_h;
      if (j >= np_h) {
        j -= np_h;
        c = rr.cos_w;
        s = rr.sin_w;
      }
    }
    out[2 * i] = c[j];
    out[2 * i + 1] = s[j];
  }
}

hipError_t launch_rope_pairs(const rotattn_rope_rot* rr, int np_t, int np_h, int np_w, float* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_rope_pairs, dim3(32), dim3(256), 0, st, *rr, np_t, np_h, np_w, out);
  return hipGetLastError();
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide amax -> (inv, scale); every thread gets both.
__device__ __forceinline__ void block_scale(float local, float* red, float& inv, float& scale) {
  const int w = ltid() >> 6;
  local = wave_max(local);
  if ((ltid() & 63) == 0) red[w] = local;
  __syncthreads();
  if (ltid() == 0) {
    float amax = red[0];
    for (int i = 1; i < kThreads / 64; ++i) amax = fmaxf(amax, red[i]);
    red[8] = amax == 0.0f ? 0.0f : 7.0f / amax;   // correctly rounded division
    red[9] = amax == 0.0f ? 0.0f : amax / 7.0f;
  }
  __syncthreads();
  inv = red[8];
  scale = red[9];
  __syncthreads();   // red[] is reused by the next reduction
}

// The code bytes of two values in bits 0-7 and 8-15: code =
// clamp(rne(fl(z inv)), -7, 7) (the + 0 turns a -0 into +0), stored as E4M3
// bytes for the FP8 layout (v_cvt_pk_fp8_f32 is exact on these integers:
// 1 = 0x38, 2 = 0x40, ..., 7 = 0x4E, sign in bit 7) or as int8 bytes.
template <bool F8>
__device__ __forceinline__ uint32_t code_pair(float z0, float z1, float inv) {
  const float q0 = __builtin_amdgcn_fmed3f(__builtin_rintf(z0 * inv), -7.0f, 7.0f) + 0.0f;
  const float q1 = __builtin_amdgcn_fmed3f(__builtin_rintf(z1 * inv), -7.0f, 7.0f) + 0.0f;
  if (F8) return __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xffffu;
  return ((uint32_t)(int)q0 & 0xffu) | (((uint32_t)(int)q1 & 0xffu) << 8);
}

typedef double v4d __attribute__((ext_vector_type(4)));

// Shape of one partition's rotation on 16x16x4 fp64 MFMA steps.
template <int DA>
struct Part {
  static constexpr int KS = (DA + 3) / 4;     // k-steps (channels, zero-padded to 4)
  static constexpr int JB = (DA + 15) / 16;   // 16-wide output blocks (zero-padded)
};

// B fragments of R_a^T: lane l holds B[k][j] = R[j][k] for k = 4 ks + l/16,
// j = 16 jb + l%16 (zero outside d_a), kept as fp32 (R is fp32-valued; the
// conversion to fp64 at each use is exact).  k_rot_to_f64 lays them out lane
// by lane (kRotFragStride floats per lane, element ks * JB + jb), so that a
// lane reads its 33 (D = 128) values with 9 16-byte loads, all in flight at
// once, instead of 33 scattered fp64 loads.
template <int DA>
__device__ __forceinline__ void load_rot_frags(const float* frag,
                                               float (&b)[Part<DA>::KS][Part<DA>::JB]) {
  constexpr int KS = Part<DA>::KS, JB = Part<DA>::JB, NV = (KS * JB + 3) / 4;
  static_assert(NV * 4 <= kRotFragStride, "fragment row fits its stride");
  const int l = ltid() & 63;
  const float4* p = (const float4*)(frag + l * kRotFragStride);
  float v[NV * 4];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float4 q = p[i];
    v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) b[ks][jb] = v[ks * JB + jb];
}

// the fragments of partition `part` (0: t, 1: h, 2: w) in the rotation scratch
__device__ __forceinline__ const float* rot_frags(const double* rot64, int part) {
  return (const float*)((const uint8_t*)rot64 + kRotFragOffset) + part * 64 * kRotFragStride;
}

// Position of token n (< N) on RoPE axis `axis`: t = n / (Hg Wg),
// h = (n / Wg) mod Hg, w = n mod Wg.  Padding tokens (n >= N) have zero rows;
// any valid table row will do for them.
__device__ __forceinline__ int axis_pos(int n, int N, int axis, int HW, int gh, int gw) {
  return n < N ? (axis == 0 ? n / HW : (axis == 1 ? (n / gw) % gh : n % gw)) : 0;
}

// The RoPE'd value of channel c (< DA) of one partition for one token: the
// token's staged fp16 row xrow (one dword per channel pair, partition start),
// its table row starts at pair trow of cs_a, the (cos, sin) pairs of the
// partition's axis (built in the library scratch by k_rope_pairs).  Even channel:
// fl(x0 c) - fl(x1 s); odd channel: fl(x0 s) + fl(x1 c).  Operands are
// selected instead of branching (negation is exact).  Channels >= DA (MFMA
// zero padding) read a clamped pair.
template <int DA>
__device__ __forceinline__ float rope_channel(const uint32_t* xrow, const float* cs_a, int trow,
                                              int c) {
  const int jp = (c >> 1) < DA / 2 ? (c >> 1) : DA / 2 - 1;
  const uint32_t pr = xrow[jp];
  const float x0 = h2f((uint16_t)(pr & 0xffffu));
  const float x1 = h2f((uint16_t)(pr >> 16));
  const float2 t = *(const float2*)(cs_a + 2 * (trow + jp));   // (cos, sin)
  const float cs = t.x, sn = t.y;
  const bool odd = (c & 1) != 0;
  const float p0 = x0 * (odd ? sn : cs);
  const float p1 = x1 * (odd ? cs : sn);
  return p0 + (odd ? p1 : -p1);
}

// RoPE + rotation of one tensor over one partition (width DA at channel offset
// off, RoPE axis `axis`) for TB groups of 16 tokens from tok0: z in the MFMA
// output layout (token tok0 + 16 tb + l/16 + 4 r, channel 16 jb + l%16 of the
// partition); returns the lane's max |z|.  xs: staged fp16 rows (kRS dwords
// per row); b: R_a^T as B fragments.
template <int DA, int TB, int kRS>
__device__ __forceinline__ float rotate_part(const uint32_t* xs, const float* cs_a,
                                             float (&b)[Part<DA>::KS][Part<DA>::JB], int off,
                                             int tok0, int n0, int N, int axis, int HW, int gh,
                                             int gw, float (&z)[TB][Part<DA>::JB][4]) {
  constexpr int KS = Part<DA>::KS, JB = Part<DA>::JB;
  const int l = ltid() & 63;
  float amax = 0.0f;
  // RoPE'd A fragments of every token group, then one MFMA chain over k in
  // which each fp64 B fragment serves all TB groups
  double av[TB][KS];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int i = tok0 + 16 * tb + (l & 15);   // this lane's A row (token in the block)
    const int pos = axis_pos(n0 + i, N, axis, HW, gh, gw);
    const uint32_t* xrow = xs + i * kRS + off / 2;
    const int trow = pos * (DA / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 4 * ks + (l >> 4);                      // channel in the partition
      const float y = rope_channel<DA>(xrow, cs_a, trow, c);
      av[tb][ks] = c < DA ? (double)y : 0.0;
    }
  }
  v4d acc[TB][JB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[tb][jb] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const double bd = (double)b[ks][jb];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        acc[tb][jb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[tb][ks], bd, acc[tb][jb], 0, 0, 0);
    }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[tb][jb][r] = (float)acc[tb][jb][r];
        amax = fmaxf(amax, fabsf(z[tb][jb][r]));
      }
  return amax;
}

// RoPE only, for rotations merged into the RoPE tables (per-pair 2x2
// rotations commute with RoPE, so R RoPE(p) = RoPE with phase offsets):
// z = y = RoPE(x) exactly as the rotating path computes its A fragments, kept
// in that layout (token tok0 + 16 tb + l%16, channel 4 ks + l/16).  Returns
// the lane's max |z|.
template <int DA, int TB, int kRS>
__device__ __forceinline__ float rope_part_a(const uint32_t* xs, const float* cs_a, int off,
                                             int tok0, int n0, int N,
                                             int axis, int HW, int gh, int gw,
                                             float (&z)[TB][Part<DA>::KS]) {
  constexpr int KS = Part<DA>::KS;
  const int l = ltid() & 63;
  float amax = 0.0f;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int i = tok0 + 16 * tb + (l & 15);
    const int pos = axis_pos(n0 + i, N, axis, HW, gh, gw);
    const uint32_t* xrow = xs + i * kRS + off / 2;
    const int trow = pos * (DA / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 4 * ks + (l >> 4);
      const float y = rope_channel<DA>(xrow, cs_a, trow, c);
      z[tb][ks] = c < DA ? y : 0.0f;
      amax = fmaxf(amax, fabsf(z[tb][ks]));
    }
  }
  return amax;
}

// Codes of rope_part_a's z (A layout) into the LDS code buffer.
template <int DA, int TB, bool F8>
__device__ __forceinline__ void quant_part_a(const float (&z)[TB][Part<DA>::KS], float inv, int off,
                                             int tok0, int8_t* codes) {
  const int l = ltid() & 63;
  constexpr int KS = Part<DA>::KS;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    int8_t* crow = codes + (tok0 + 16 * tb + (l & 15)) * kCodeStride + off;
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      const uint32_t pr = code_pair<F8>(z[tb][ks], ks + 1 < KS ? z[tb][ks + 1] : 0.0f, inv);
      const int c = 4 * ks + (l >> 4);
      if (c < DA) crow[c] = (int8_t)pr;
      if (ks + 1 < KS && c + 4 < DA) crow[c + 4] = (int8_t)(pr >> 8);
    }
  }
}

// Codes of rotate_part's z (MFMA output layout) into the LDS code buffer
// ([token][channel], kCodeStride bytes per row).
template <int DA, int TB, bool F8>
__device__ __forceinline__ void quant_part(const float (&z)[TB][Part<DA>::JB][4], float inv,
                                           int off, int tok0, int8_t* codes) {
  const int l = ltid() & 63;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int jb = 0; jb < Part<DA>::JB; ++jb) {
      const int j = 16 * jb + (l & 15);
      if (j < DA) {
        int8_t* cp = codes + (tok0 + 16 * tb + (l >> 4)) * kCodeStride + off + j;
        const uint32_t p01 = code_pair<F8>(z[tb][jb][0], z[tb][jb][1], inv);
        const uint32_t p23 = code_pair<F8>(z[tb][jb][2], z[tb][jb][3], inv);
        cp[0] = (int8_t)p01;                      // rows 4 r further down for r = 0..3
        cp[4 * kCodeStride] = (int8_t)(p01 >> 8);
        cp[8 * kCodeStride] = (int8_t)p23;
        cp[12 * kCodeStride] = (int8_t)(p23 >> 8);
      }
    }
}

// V of a block: thread (token n = t mod 128, half h = t / 128) holds channels
// [h D/2, (h+1) D/2) of its token; block amax; codes transposed into codesT
// ([channel][token], kCodeStride bytes per channel row).  codesT may be the
// staging buffer itself: every row is read before the reduction's barriers.
template <int D, bool F8>
__device__ __forceinline__ void v_codes(const uint32_t* xs, float* red, int8_t* codesT,
                                        float& scale_out) {
  constexpr int kRS = D / 2 + 1;
  constexpr int C = D / 2;   // channels per thread
  const int n = ltid() & (kBlock - 1), h = ltid() / kBlock;
  const uint32_t* xrow = xs + n * kRS + h * (C / 2);
  float x[C];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < C / 2; ++j) {
    const uint32_t pr = xrow[j];
    x[2 * j] = h2f((uint16_t)(pr & 0xffffu));
    x[2 * j + 1] = h2f((uint16_t)(pr >> 16));
    amax = fmaxf(amax, fmaxf(fabsf(x[2 * j]), fabsf(x[2 * j + 1])));
  }
  float inv, scale;
  block_scale(amax, red, inv, scale);
  int8_t* cp = codesT + h * C * kCodeStride + n;
#pragma unroll
  for (int r = 0; r < C; r += 2) {
    const uint32_t pr = code_pair<F8>(x[r], x[r + 1], inv);
    cp[r * kCodeStride] = (int8_t)pr;
    cp[(r + 1) * kCodeStride] = (int8_t)(pr >> 8);
  }
  scale_out = scale;
}

// Stage 128 fp16 rows (tokens n0..n0+127 of one head, row_stride elements
// apart) into xs, kRS dwords per row (the odd stride keeps per-token reads
// conflict-free), zero rows for tokens >= N.  Each wave instruction moves one
// row straight from memory into LDS (global_load_lds, lane L -> dword L of the
// row): no registers, no waits here.  The caller waits with wait_tiles()
// before the barrier that publishes the rows.
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* src, int64_t row_stride, int n0, int N,
                                          uint32_t* xs) {
  constexpr int kRS = D / 2 + 1;
  constexpr int kW = kThreads / 64;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int lane = ltid() & 63;
  const int w = __builtin_amdgcn_readfirstlane(ltid() >> 6);
#pragma unroll 1
  for (int r = w; r < kBlock; r += kW) {
    if (n0 + r < N) {
      if (lane < D / 2)
        __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)(n0 + r) * row_stride + 2 * lane),
                                         (lds_ptr)(xs + r * kRS), 4, 0, 0);
    } else if (lane < D / 2) {
      xs[r * kRS + lane] = 0u;
    }
  }
}

__device__ __forceinline__ void wait_tiles() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Coalesced store of all 128 staged fp16 rows (rows past N are zero) into a
// padded [N_pad][D] buffer.
template <int D>
__device__ __forceinline__ void store_tile_all(uint16_t* dst, int n0, const uint32_t* xs) {
  constexpr int kChunks = D / 8;
  constexpr int kRS = D / 2 + 1;
  for (int i = ltid(); i < kBlock * kChunks; i += kThreads) {
    const int r = i / kChunks, c = i % kChunks;
    const uint32_t* s_ = xs + r * kRS + 4 * c;
    *(uint4*)(dst + (size_t)(n0 + r) * D + 8 * c) = uint4{s_[0], s_[1], s_[2], s_[3]};
  }
}

// The block's staged fp16 V rows (rows past N zero) -> its two 64-key V^T
// tiles, [D][64] each, in the operand order of the fp16 P.V product: position
// 32s + 4c + i holds key 32s + 4c' + i, c' = c with bits 0 and 1 swapped.
template <int D>
__device__ __forceinline__ void store_vt_tiles(const uint32_t* xs, uint16_t* dst) {
  constexpr int kRS = D / 2 + 1;
  for (int item = ltid(); item < 2 * D * 8; item += kThreads) {
    const int tl = item / (D * 8), d = (item / 8) % D, j = item % 8;   // 8 positions per item
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t hv[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int pos = 8 * j + e + f;                   // 0..63
        const int s = pos >> 5, pc = (pos >> 2) & 7, i = pos & 3;
        const int c = (pc & 4) | ((pc & 1) << 1) | ((pc >> 1) & 1);
        const int key = 64 * tl + 32 * s + 4 * c + i;    // token within the block
        hv[f] = (xs[key * kRS + (d >> 1)] >> (16 * (d & 1))) & 0xffffu;
      }
      w[e / 2] = hv[0] | (hv[1] << 16);
    }
    *(uint4*)(dst + ((size_t)tl * D + d) * 64 + 8 * j) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// Q/K codes (LDS, [token][channel]) -> packed rows [128][D/2] in global memory.
template <int D>
__device__ __forceinline__ void store_qk_codes(const int8_t* codes, uint8_t* dst) {
  constexpr int kDw = D / 8;   // packed dwords per token
  for (int i = ltid(); i < kBlock * kDw; i += kThreads) {
    const int n = i / kDw, g = i % kDw;
    const uint32_t lo = *(const uint32_t*)(codes + n * kCodeStride + 8 * g);
    const uint32_t hi = *(const uint32_t*)(codes + n * kCodeStride + 8 * g + 4);
    *(uint32_t*)(dst + (size_t)n * (D / 2) + 4 * g) = pack_nibbles(lo, hi);
  }
}

// FP8 layout: Q/K code bytes (LDS, [token][channel]) -> rows [128][D].
template <int D>
__device__ __forceinline__ void store_qk_codes_f8(const int8_t* codes, uint8_t* dst) {
  constexpr int kDw = D / 4;
  for (int i = ltid(); i < kBlock * kDw; i += kThreads) {
    const int n = i / kDw, g = i % kDw;
    *(uint32_t*)(dst + (size_t)n * D + 4 * g) = *(const uint32_t*)(codes + n * kCodeStride + 4 * g);
  }
}

// FP8 layout: V code bytes (LDS, [channel][token]) -> V^T block [D][128], each
// 64-key half in the operand order of the P.V product with P as FP6 (byte
// 32h + j of a half holds key 32h + 8((j%16)/4) + 4(j/16) + j%4).  Dwords move
// whole: j%4 is the byte.
template <int D>
__device__ __forceinline__ void store_v_codes_f8(const int8_t* codesT, uint8_t* dst) {
  for (int i = ltid(); i < D * 32; i += kThreads) {
    const int d = i / 32, q = i % 32;                 // output dword q of row d
    const int c = q / 16, h = (q / 8) & 1, j = 4 * (q & 7);
    const int key = 64 * c + 32 * h + 8 * ((j % 16) / 4) + 4 * (j / 16);
    *(uint32_t*)(dst + (size_t)d * 128 + 4 * q) = *(const uint32_t*)(codesT + d * kCodeStride + key);
  }
}

// FP6 E2M3 fields of four int8 codes in [-7, 7], one code per byte in and one
// field per byte out: sign in bit 5, and the magnitudes 0..7 are exact E2M3
// values (exponent bias 1): 0, 1.0, 2.0, 1.5 x 2, 4.0, 1.25 x 4, 1.5 x 4,
// 1.75 x 4 have the bits 0, 8, 16, 20, 24, 26, 28, 30, looked up per byte
// with v_perm_b32 (selector bytes 0..3 pick from the low table dword, 4..7
// from the high one).
__device__ __forceinline__ uint32_t e2m3_fields4(uint32_t c) {
  const uint32_t neg = (c >> 7) & 0x01010101u;
  const uint32_t flip = (neg << 7) - neg;                         // 0x7f in negative bytes
  const uint32_t mag = ((c ^ flip) + neg) & 0x07070707u;         // |c| per byte
  return __builtin_amdgcn_perm(0x1e1c1a18u, 0x14100800u, mag) | (neg << 5);
}

// 32 fields (one per byte of f[0..7], field 4i + j in byte j of f[i]) packed
// six bits each, field k at bits 6k..6k+5 of the 192-bit little-endian word
// out[0..5]: the FP6 operand of one lane half of a 32x32x64 f8f6f4 MFMA.
__device__ __forceinline__ void pack_fields32(const uint32_t (&f)[8], uint32_t (&out)[6]) {
  uint32_t w[8];   // 24 bits: four fields
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t x = f[i];
    w[i] = (x & 0x3fu) | ((x >> 2) & 0xfc0u) | ((x >> 4) & 0x3f000u) | ((x >> 6) & 0xfc0000u);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    out[3 * h] = w[4 * h] | (w[4 * h + 1] << 24);
    out[3 * h + 1] = (w[4 * h + 1] >> 8) | (w[4 * h + 2] << 16);
    out[3 * h + 2] = (w[4 * h + 2] >> 16) | (w[4 * h + 3] << 8);
  }
}

// FP6 layout: Q/K int8 codes (LDS, [token][channel]) -> rows [128][D], each
// 32-channel group in 32 bytes: channel 32g + k in field k of the group's 24
// FP6 bytes, then 8 zero bytes.
template <int D>
__device__ __forceinline__ void store_qk_codes_f6(const int8_t* codes, uint8_t* dst) {
  constexpr int kG = D / 32;   // groups per token
  for (int i = ltid(); i < kBlock * kG; i += kThreads) {
    const int n = i / kG, g = i % kG;
    const uint32_t* src = (const uint32_t*)(codes + n * kCodeStride + 32 * g);
    uint32_t f[8], o[6];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = e2m3_fields4(src[j]);
    pack_fields32(f, o);
    uint8_t* d = dst + (size_t)n * D + 32 * g;
    *(uint4*)d = uint4{o[0], o[1], o[2], o[3]};
    *(uint4*)(d + 16) = uint4{o[4], o[5], 0u, 0u};
  }
}

// FP6 layout: V int8 codes (LDS, [channel][token]) -> V^T block [D][128], each
// row in four 32-byte groups g = 2c + h (64-key chunk c, MFMA lane half h) of
// 24 FP6 bytes and 8 zero bytes.  Field k of group (c, h) holds key
// 64c + 32(k/16) + 8((k%16)/4) + 4h + k%4: the key that field k of the P^T
// operand (FP6, taken from the S^T accumulator layout) holds in lane half h.
// The fields come four at a time: k%4 is the byte of a code dword.
template <int D>
__device__ __forceinline__ void store_v_codes_f6(const int8_t* codesT, uint8_t* dst) {
  for (int i = ltid(); i < D * 4; i += kThreads) {
    const int d = i / 4, g = i % 4, c = g / 2, h = g % 2;
    const int8_t* row = codesT + d * kCodeStride + 64 * c + 4 * h;
    uint32_t f[8], o[6];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = e2m3_fields4(*(const uint32_t*)(row + 32 * (j / 4) + 8 * (j % 4)));
    pack_fields32(f, o);
    uint8_t* dp = dst + (size_t)d * 128 + 32 * g;
    *(uint4*)dp = uint4{o[0], o[1], o[2], o[3]};
    *(uint4*)(dp + 16) = uint4{o[4], o[5], 0u, 0u};
  }
}

// V codes (LDS, [channel][token]) -> packed V^T block [D][64] in global memory.
template <int D>
__device__ __forceinline__ void store_v_codes(const int8_t* codesT, uint8_t* dst) {
  for (int i = ltid(); i < D * 16; i += kThreads) {
    const int d = i / 16, g = i % 16;
    const uint32_t lo = *(const uint32_t*)(codesT + d * kCodeStride + 8 * g);
    const uint32_t hi = *(const uint32_t*)(codesT + d * kCodeStride + 8 * g + 4);
    *(uint32_t*)(dst + (size_t)d * 64 + 4 * g) = pack_nibbles(lo, hi);
  }
}

// One tensor of a head that is not a fallback head (s = 0: Q, 1: K) from its
// 128 staged fp16 rows xs (kRS dwords per row, rows past N zero).  Wave w owns
// tokens 32w..32w+31 of the block in every partition: RoPE + rotation on the
// MFMA (or RoPE alone), block amax, codes into xs (every wave is past its last
// read of the rows once the reduction's barriers are passed), coalesced
// store, block scale.  mid() runs right after the reduction, before the codes
// are made: the prologue requests V's rows there.
template <int D, int D0, int D1, int LAY, bool ROT, class Mid>
__device__ __forceinline__ void quant_qk_tile(const PrologueArgs& a, uint32_t* xs, float* red,
                                              int s, int blk, int bh, Mid mid) {
  constexpr int kRS = D / 2 + 1;
  constexpr int TB = kBlock / 16 / (kThreads / 64);   // 16-token groups per wave
  // LDS codes: E4M3 bytes for the FP8 layout, int8 for the others
  constexpr bool F8 = LAY == ROTATTN_LAYOUT_FP8;
  const int w = ltid() >> 6;
  const int tok0 = 16 * TB * w;
  const int n0 = blk * kBlock;
  const int HW = a.grid_h * a.grid_w;
  const size_t pad_row = ((size_t)bh * a.NB + blk) * kBlock;   // first code row of this block
  int8_t* codes = (int8_t*)xs;
  float inv, scale;
  // the table reads are the same for Q and K; an opaque zero offset per
  // tensor keeps the compiler from loading them once and holding them in
  // registers across both tensors
  int zero = 0;
  asm volatile("" : "+s"(zero));
  const float *cs_t = a.cs_t + zero, *cs_h = a.cs_h + zero, *cs_w = a.cs_w + zero;
  if (ROT) {
    // R_a^T of each partition as B fragments, loaded (from cache) just before
    // its use; rotation matrices in fp64 [k][r]: t at 0, h at D0^2, w at
    // D0^2 + D1^2
    float z0[TB][Part<D0>::JB][4], z1[TB][Part<D1>::JB][4], z2[TB][Part<D1>::JB][4];
    float amax;
    {
      float b[Part<D0>::KS][Part<D0>::JB];
      load_rot_frags<D0>(rot_frags(a.rot64, 0) + zero, b);   // read again per tensor, not held
      amax = rotate_part<D0, TB, kRS>(xs, cs_t, b, 0, tok0, n0, a.N, 0, HW, a.grid_h,
                                      a.grid_w, z0);
    }
    {
      float b[Part<D1>::KS][Part<D1>::JB];
      load_rot_frags<D1>(rot_frags(a.rot64, 1) + zero, b);
      amax = fmaxf(amax, rotate_part<D1, TB, kRS>(xs, cs_h, b, D0, tok0, n0, a.N, 1,
                                                  HW, a.grid_h, a.grid_w, z1));
    }
    {
      float b[Part<D1>::KS][Part<D1>::JB];
      load_rot_frags<D1>(rot_frags(a.rot64, 2) + zero, b);
      amax = fmaxf(amax, rotate_part<D1, TB, kRS>(xs, cs_w, b, D0 + D1, tok0, n0,
                                                  a.N, 2, HW, a.grid_h, a.grid_w, z2));
    }
    block_scale(amax, red, inv, scale);
    mid();
    quant_part<D0, TB, F8>(z0, inv, 0, tok0, codes);
    quant_part<D1, TB, F8>(z1, inv, D0, tok0, codes);
    quant_part<D1, TB, F8>(z2, inv, D0 + D1, tok0, codes);
  } else {
    float z0[TB][Part<D0>::KS], z1[TB][Part<D1>::KS], z2[TB][Part<D1>::KS];
    float amax = rope_part_a<D0, TB, kRS>(xs, cs_t, 0, tok0, n0, a.N, 0, HW,
                                          a.grid_h, a.grid_w, z0);
    amax = fmaxf(amax, rope_part_a<D1, TB, kRS>(xs, cs_h, D0, tok0, n0, a.N, 1, HW,
                                                a.grid_h, a.grid_w, z1));
    amax = fmaxf(amax, rope_part_a<D1, TB, kRS>(xs, cs_w, D0 + D1, tok0, n0, a.N,
                                                2, HW, a.grid_h, a.grid_w, z2));
    block_scale(amax, red, inv, scale);
    mid();
    quant_part_a<D0, TB, F8>(z0, inv, 0, tok0, codes);
    quant_part_a<D1, TB, F8>(z1, inv, D0, tok0, codes);
    quant_part_a<D1, TB, F8>(z2, inv, D0 + D1, tok0, codes);
  }
  __syncthreads();
  if (LAY == ROTATTN_LAYOUT_FP8)
    store_qk_codes_f8<D>(codes, (s == 0 ? a.q4 : a.k4) + pad_row * D);
  else if (LAY == ROTATTN_LAYOUT_FP6)
    store_qk_codes_f6<D>(codes, (s == 0 ? a.q4 : a.k4) + pad_row * D);
  else
    store_qk_codes<D>(codes, (s == 0 ? a.q4 : a.k4) + pad_row * (D / 2));
  if (ltid() == 0) {
    if (s == 0)
      a.q_scale_l2[(size_t)bh * a.NB + blk] = scale * a.kappa;
    else
      a.k_scale[(size_t)bh * a.NB + blk] = scale;
  }
}

// V of a head that is not a fallback head, from its staged fp16 rows xs:
// block amax, codes (in place), stored transposed, block scale.
template <int D, int LAY>
__device__ __forceinline__ void quant_v_tile(const PrologueArgs& a, uint32_t* xs, float* red,
                                             int blk, int bh) {
  int8_t* codes = (int8_t*)xs;
  float scale;
  v_codes<D, LAY == ROTATTN_LAYOUT_FP8>(xs, red, codes, scale);
  __syncthreads();
  if (LAY == ROTATTN_LAYOUT_FP8)
    store_v_codes_f8<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 128);
  else if (LAY == ROTATTN_LAYOUT_FP6)
    store_v_codes_f6<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 128);
  else
    store_v_codes<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 64);
  if (ltid() == 0) a.v_scale[(size_t)bh * a.NB + blk] = scale;
}

// A head that is not a fallback head: Q and K staged together, each tensor
// inlined on its own (straight-line code, so nothing is hoisted across the two
// tensors and kept live); V's rows are requested during the K pass, once every
// wave is done with the Q codes in stage_q, and stream in while K is
// quantized and stored.
template <int D, int D0, int D1, int LAY, bool ROT>
__device__ __forceinline__ void prologue_qk(const PrologueArgs& a, uint32_t* stage_q,
                                            uint32_t* stage_k, float* red, int blk, int bh) {
  const int n0 = blk * kBlock;
  const int64_t head_in = a.in.head_offset(bh, a.H);
  load_tile<D>(a.q + head_in, a.in.token, n0, a.N, stage_q);
  load_tile<D>(a.k + head_in, a.in.token, n0, a.N, stage_k);
  wait_tiles();
  __syncthreads();
  quant_qk_tile<D, D0, D1, LAY, ROT>(a, stage_q, red, 0, blk, bh, [] {});
  quant_qk_tile<D, D0, D1, LAY, ROT>(a, stage_k, red, 1, blk, bh, [&] {
    load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage_q);
  });
  __syncthreads();
  // V: staged in the Q buffer, codes in place
  wait_tiles();
  __syncthreads();
  quant_v_tile<D, LAY>(a, stage_q, red, blk, bh);
}

// Fallback head, RoPE of one staged tensor in place: thread (token n, half h)
// applies RoPE to partition t (h = 0) or partitions h and w (h = 1) of its
// token's row in fp32 and writes the fp16 pairs back once every thread has
// read its row.
template <int D, int D0, int D1>
__device__ __forceinline__ void rope_fallback(const PrologueArgs& a, uint32_t* xs, int n0) {
  constexpr int kRS = D / 2 + 1;
  constexpr int NY = D0 > 2 * D1 ? D0 : 2 * D1;
  const int n = ltid() & (kBlock - 1);
  const int half = __builtin_amdgcn_readfirstlane(ltid() / kBlock);
  const int HW = a.grid_h * a.grid_w;
  uint32_t* xrow = xs + n * kRS;
  float y[NY];
  if (half == 0) {
    float yt[D0];
    rope_part<D0>(xrow, a.cos_t, a.sin_t, axis_pos(n0 + n, a.N, 0, HW, a.grid_h, a.grid_w), 0, yt);
#pragma unroll
    for (int i = 0; i < D0; ++i) y[i] = yt[i];
  } else {
    float yh[D1], yw[D1];
    rope_part<D1>(xrow, a.cos_h, a.sin_h, axis_pos(n0 + n, a.N, 1, HW, a.grid_h, a.grid_w), D0, yh);
    rope_part<D1>(xrow, a.cos_w, a.sin_w, axis_pos(n0 + n, a.N, 2, HW, a.grid_h, a.grid_w),
                  D0 + D1, yw);
#pragma unroll
    for (int i = 0; i < D1; ++i) {
      y[i] = yh[i];
      y[D1 + i] = yw[i];
    }
  }
  __syncthreads();   // every thread has read its inputs before any row is overwritten
  if (half == 0) {
#pragma unroll
    for (int j = 0; j < D0 / 2; ++j)
      xrow[j] = (uint32_t)f2h(y[2 * j]) | ((uint32_t)f2h(y[2 * j + 1]) << 16);
  } else {
#pragma unroll
    for (int j = 0; j < D1; ++j)
      xrow[D0 / 2 + j] = (uint32_t)f2h(y[2 * j]) | ((uint32_t)f2h(y[2 * j + 1]) << 16);
  }
}

// Fallback head: RoPE'd fp16 Q and K into the padded q_rope/k_rope rows, then
// V^T tiles for the fp16 attention.
template <int D, int D0, int D1>
__device__ __forceinline__ void prologue_fallback(const PrologueArgs& a, uint32_t* stage_q,
                                                  uint32_t* stage_k, int blk, int bh) {
  const int n0 = blk * kBlock;
  const int64_t head_in = a.in.head_offset(bh, a.H);
  const size_t head_pad = (size_t)bh * a.NB * kBlock;
  load_tile<D>(a.q + head_in, a.in.token, n0, a.N, stage_q);
  load_tile<D>(a.k + head_in, a.in.token, n0, a.N, stage_k);
  wait_tiles();
  __syncthreads();
  rope_fallback<D, D0, D1>(a, stage_q, n0);
  rope_fallback<D, D0, D1>(a, stage_k, n0);
  __syncthreads();
  store_tile_all<D>(a.q_rope + head_pad * D, n0, stage_q);
  store_tile_all<D>(a.k_rope + head_pad * D, n0, stage_k);
  __syncthreads();
  load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage_q);
  wait_tiles();
  __syncthreads();
  store_vt_tiles<D>(stage_q, a.v_t + (head_pad + n0) * D);
}

// Staging for the FP16 attention on caller buffers: already RoPE'd fp16 Q', K'
// and V of the selected heads (read through their strides) -> zero-padded
// [N_pad][D] rows of Q' and K' and the V^T tiles of the FP16 P.V operand,
// the layout the FP16 attention kernel reads.  One work-group per (128-token
// block, head of the chunk [bh0, bh0 + gridDim.y)); buffers are indexed by
// the head's place in the chunk.
template <int D>
__global__ __launch_bounds__(kThreads) void k_stage_fp16(StageArgs a) {
  constexpr int kRS = D / 2 + 1;
  __shared__ __align__(16) uint32_t stage[kBlock * kRS];
  const int blk = blockIdx.x, lh = blockIdx.y, bh = a.bh0 + lh;
  if (!a.run.test(bh)) return;
  const int n0 = blk * kBlock;
  const int64_t head_in = a.in.head_offset(bh, a.H);
  const size_t head_pad = (size_t)lh * a.NB * kBlock;
  const uint16_t* src[2] = {a.q, a.k};
  uint16_t* dst[2] = {a.q_pad, a.k_pad};
  for (int s = 0; s < 2; ++s) {
    load_tile<D>(src[s] + head_in, a.in.token, n0, a.N, stage);
    wait_tiles();
    __syncthreads();
    store_tile_all<D>(dst[s] + head_pad * D, n0, stage);
    __syncthreads();
  }
  load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage);
  wait_tiles();
  __syncthreads();
  store_vt_tiles<D>(stage, a.v_t + (head_pad + n0) * D);
}

hipError_t launch_stage_fp16(int D, int nbh, const StageArgs& a, hipStream_t st) {
  dim3 grid(a.NB, nbh);
  if (D == 128)
    hipLaunchKernelGGL(k_stage_fp16<128>, grid, dim3(kThreads), 0, st, a);
  else if (D == 64)
    hipLaunchKernelGGL(k_stage_fp16<64>, grid, dim3(kThreads), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// One work-group per (128-token block, head), 4 waves (one per SIMD): two
// work-groups share a CU (LDS), so one group's MFMA phase overlaps the other's
// memory phases.
template <int D, int D0, int D1, int LAY, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_prologue(PrologueArgs a) {
  static_assert(D0 + 2 * D1 == D, "split must be (D0, D1, D1)");
  constexpr int kRS = D / 2 + 1;   // staged fp16 row, in dwords
  static_assert(kBlock * kCodeStride <= kBlock * kRS * 4, "codes fit in a staging buffer");
  static_assert(D * kCodeStride <= kBlock * kRS * 4, "transposed codes fit in a staging buffer");
  static_assert(Part<D0>::JB == Part<D1>::JB, "partitions share the output block count");
  // two buffers of 128 staged fp16 rows (Q and K; later V and the codes)
  __shared__ __align__(16) uint32_t stage_q[kBlock * kRS];
  __shared__ __align__(16) uint32_t stage_k[kBlock * kRS];
  __shared__ float red[16];
  const int blk = blockIdx.x, bh = blockIdx.y;
  if (a.fallback.test(bh))
    prologue_fallback<D, D0, D1>(a, stage_q, stage_k, blk, bh);
  else
    prologue_qk<D, D0, D1, LAY, ROT>(a, stage_q, stage_k, red, blk, bh);
}

template <int D, int D0, int D1, int LAY>
static void launch_prologue_l(bool rot, dim3 grid, const PrologueArgs& a, hipStream_t st) {
  if (rot)
    hipLaunchKernelGGL((k_prologue<D, D0, D1, LAY, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_prologue<D, D0, D1, LAY, false>), grid, dim3(kThreads), 0, st, a);
}

template <int D, int D0, int D1>
static void launch_prologue_t(int layout, bool rot, dim3 grid, const PrologueArgs& a,
                              hipStream_t st) {
  if (layout == ROTATTN_LAYOUT_FP8)
    launch_prologue_l<D, D0, D1, ROTATTN_LAYOUT_FP8>(rot, grid, a, st);
  else if (layout == ROTATTN_LAYOUT_FP6)
    launch_prologue_l<D, D0, D1, ROTATTN_LAYOUT_FP6>(rot, grid, a, st);
  else
    launch_prologue_l<D, D0, D1, ROTATTN_LAYOUT_PACKED>(rot, grid, a, st);
}

hipError_t launch_prologue(int D, int dt, int BH, int layout, bool rot, const PrologueArgs& a,
                           hipStream_t st) {
  dim3 grid(a.NB, BH);
  if (D == 128 && dt == 44)
    launch_prologue_t<128, 44, 42>(layout, rot, grid, a, st);
  else if (D == 64 && dt == 24)
    launch_prologue_t<64, 24, 20>(layout, rot, grid, a, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------- QKV projection + prologue
//
// The step before the attention in a DiT block, fused: the QKV projection of
// the block's input computes one 128-token x 128-channel tile (one head's Q,
// K or V for one token block) per work-group, and the tile, rounded to fp16
// in LDS, goes straight into the prologue's work above instead of through
// HBM.  Projection: C^T = W_rows X_tokens^T on v_mfma_f32_32x32x16_f16 with
// fp32 accumulation (W rows and X rows are both contiguous along the
// reduction), 4 waves of 64 channels x 64 tokens.  Both tiles stream through
// LDS in 64-deep stages (global_load_lds into XOR-swizzled rows), double
// buffered, one barrier per stage.  + bias in fp32, one rounding to fp16; each
// lane then holds 4 consecutive channels of one token per 32x32 block: two
// dword writes of the staged row.

constexpr int kGK = 64;                      // reduction depth of one stage
constexpr int kGRow = kGK * 2;               // bytes of a tile row in a stage
constexpr int kGTile = 128 * kGRow;          // bytes of one 128-row tile of a stage
constexpr int kGStage = 2 * kGTile;          // W tile, then X tile

// XOR swizzle of the 16-byte chunks of a 128-byte row: the 16 rows a
// ds_read_b128 reads together land on 16 different chunk columns of the 64
// banks (two rows per 256-byte bank row).
__device__ __forceinline__ int gswz(int row) { return (row >> 1) & 7; }

template <int D, int D0, int D1, int LAY, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_qkv_proj_prologue(QkvProjArgs a) {
  static_assert(D == 128, "one 128-channel head per work-group tile");
  constexpr int kRS = D / 2 + 1;
  constexpr int kStaged = kBlock * kRS * 4;            // bytes of the staged fp16 tile
  static_assert(kStaged >= kGStage, "stage 0 sits inside the staging buffer");
  // stage 0 in the buffer that later holds the staged tile, stage 1 in an
  // array of its own: separate arrays let the compiler see that the next
  // stage's loads into one never alias the operand reads of the other, so it
  // does not wait for them before those reads
  __shared__ __align__(16) uint8_t staged[kStaged];
  __shared__ __align__(16) uint8_t stage1[kGStage];
  __shared__ float red[16];
  typedef __attribute__((address_space(3))) void* lds_ptr;

  // tile of this work-group: dispatch is round-robin over the 8 XCDs, so
  // ids L, L+8, L+16, ... share an XCD (and its L2); each XCD works through
  // groups of 64 tiles = 8 token blocks x 8 (tensor, head) pairs
  const int H = a.p.H, NB = a.p.NB, N = a.p.N;
  int tb, ht;                                   // token block over all batches, (tensor, head) pair
  if (a.last_block_only) {
    // the blocks the 256 x 256 kernel leaves over: the last of each batch entry
    const int L = blockIdx.x;
    if (L >= a.B * 3 * H) return;
    tb = (L / (3 * H)) * NB + NB - 1;
    ht = L % (3 * H);
  } else {
    const int L = blockIdx.x;
    const int S = (L / 512) * 8 + (L % 8);      // group
    const int r = (L / 8) % 64;                 // tile within the group
    if (S >= a.SBT * a.SHT) return;
    tb = (S % a.SBT) * 8 + (r % 8);
    ht = (S / a.SBT) * 8 + (r / 8);
    if (tb >= a.B * NB || ht >= 3 * H) return;
  }
  const int b = tb / NB, blk = tb % NB, t = ht / H, h = ht % H;
  const int bh = b * H + h, n0 = blk * kBlock;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int wm = w & 1, wn = w >> 1;            // wave's 64 channels, 64 tokens
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // stage loads: wave instruction i (0..3) fills the 1 KiB window 4i + w of a
  // tile, rows 8 (4i + w) + lane/8; physical chunk lane%8 holds logical chunk
  // (lane%8) ^ gswz(row), and rows 32 apart share the key, so instruction i's
  // offset is instruction 0's plus 32 rows
  const int lrow = 8 * w + lane / 8;
  const int lchunk = (lane % 8) ^ gswz(lrow);
  const size_t wrow_bytes = (size_t)a.C * 2;
  const uint8_t* wbase = (const uint8_t*)(a.w + (size_t)ht * D * a.C);
  const uint32_t woff = (uint32_t)(lrow * wrow_bytes) + 16 * lchunk;
  const uint8_t* xbase = (const uint8_t*)(a.x + (int64_t)b * a.x_batch + (int64_t)n0 * a.x_token);
  const int rmax = (N - n0 < kBlock ? N - n0 : kBlock) - 1;   // rows past N read the last valid row
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = lrow + 32 * i;
    xoff[i] = (uint32_t)((int64_t)(row < rmax ? row : rmax) * a.x_token * 2) + 16 * lchunk;
  }
  // uniform base in an SGPR pair + 32-bit lane offset (the saddr form); the
  // offsets are made opaque per stage so that the loop does not keep per-lane
  // 64-bit pointers in registers
  auto gload = [&](int it, uint8_t* slot) {
    uint32_t wo = woff, xo0 = xoff[0], xo1 = xoff[1], xo2 = xoff[2], xo3 = xoff[3];
    asm volatile("" : "+v"(wo), "+v"(xo0), "+v"(xo1), "+v"(xo2), "+v"(xo3));
    const uint32_t xo[4] = {xo0, xo1, xo2, xo3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* wb = wbase + (size_t)it * kGRow + (size_t)32 * i * wrow_bytes;
      const uint8_t* xb = xbase + (size_t)it * kGRow;
      asm volatile("" : "+s"(wb), "+s"(xb));
      __builtin_amdgcn_global_load_lds((const void*)(wb + wo),
                                       (lds_ptr)(slot + (4 * i + wu) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(xb + xo[i]),
                                       (lds_ptr)(slot + kGTile + (4 * i + wu) * 1024), 16, 0, 0);
    }
  };

  // operand reads: logical chunk 2 ks + hh of row r sits at byte
  // 16 ((2 ks + hh) ^ gswz(r)) = (16 (hh ^ gswz(r))) ^ 32 ks of the row;
  // rows 32 apart share the key
  uint32_t xa = (64 * wm + col) * kGRow + 16 * (hh ^ gswz(64 * wm + col));
  uint32_t xb = kGTile + (64 * wn + col) * kGRow + 16 * (hh ^ gswz(64 * wn + col));
  asm volatile("" : "+v"(xa), "+v"(xb));
  v16f acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = v16f{0.0f};
  const int kIters = a.C / kGK;

  // stage it from `cur`: request stage it+1 into `next` (last read in
  // iteration it-1, before the barrier), 16 MFMAs, wait, barrier
  auto step = [&](int it, const uint8_t* cur, uint8_t* next) {
    if (it + 1 < kIters) gload(it + 1, next);
    // all 16 operand reads of the stage first, so that later k-steps' reads
    // are in flight while the first MFMAs run
    v8h fa[kGK / 16][2], fb[kGK / 16][2];
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        fa[ks][m] = *(const v8h*)(cur + ((xa + 32 * kGRow * m) ^ (32 * ks)));
        fb[ks][m] = *(const v8h*)(cur + ((xb + 32 * kGRow * m) ^ (32 * ks)));
      }
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[ks][mi], fb[ks][ni], acc[mi][ni],
                                                                0, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  gload(0, staged);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll 1
  for (int it = 0; it < kIters; it += 2) {
    step(it, staged, stage1);
    if (it + 1 < kIters) step(it + 1, stage1, staged);
  }

  // epilogue 1: + bias, fp16, staged rows (token n: kRS dwords, channel pairs);
  // the last barrier above has every wave past its last stage read and every
  // load landed
  uint32_t* xs = (uint32_t*)staged;
  const int nvalid = N - n0;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int tok = 64 * wn + 32 * ni + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 64 * wm + 32 * mi + 8 * g + 4 * hh;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[mi][ni][4 * g + e];
          if (a.bias) v[e] += h2f(a.bias[(size_t)ht * D + c0 + e]);
        }
        uint32_t p0 = (uint32_t)f2h(v[0]) | ((uint32_t)f2h(v[1]) << 16);
        uint32_t p1 = (uint32_t)f2h(v[2]) | ((uint32_t)f2h(v[3]) << 16);
        if (tok >= nvalid) p0 = p1 = 0u;
        xs[tok * kRS + c0 / 2] = p0;
        xs[tok * kRS + c0 / 2 + 1] = p1;
      }
    }
  __syncthreads();
  const size_t BH = (size_t)a.B * H, N_pad = (size_t)NB * kBlock;
  if (a.qkv_out) store_tile_all<D>(a.qkv_out + ((size_t)t * BH + bh) * N_pad * D, n0, xs);

  // epilogue 2: the prologue's work on the staged tile
  if (a.p.fallback.test(bh)) {
    if (t < 2) {
      rope_fallback<D, D0, D1>(a.p, xs, n0);
      __syncthreads();
      store_tile_all<D>((t == 0 ? a.p.q_rope : a.p.k_rope) + (size_t)bh * N_pad * D, n0, xs);
    } else {
      store_vt_tiles<D>(xs, a.p.v_t + ((size_t)bh * N_pad + n0) * D);
    }
  } else if (t < 2) {
    quant_qk_tile<D, D0, D1, LAY, ROT>(a.p, xs, red, t, blk, bh, [] {});
  } else {
    quant_v_tile<D, LAY>(a.p, xs, red, blk, bh);
  }
}

// The same projection on a 256-channel x 256-token work-group tile: two
// (tensor, head) pairs 2j, 2j+1 (rows 256 j .. 256 j + 255 of W, contiguous) x
// two token blocks 2i, 2i+1 of one batch entry, 8 waves of 64 channels x 128
// tokens.  A 64-deep stage brings 64 KiB for 8.4 MFLOP, half the bytes per
// flop of the 128 x 128 tile, whose feed is bounded by the L2.  One
// work-group per CU (two buffers of staged + packed tile size, each holding
// one stage of the double-buffered projection).  Epilogue in two rounds on the
// two halves of the work-group (waves 0-3: token block 2i, waves 4-7: 2i+1),
// each half running one prologue unit: round one the first (tensor, head),
// whose fp16 tiles go straight to the staged layout, round two the second,
// whose tiles wait packed (XOR-swizzled rows) beside them.  Both halves of a
// round work on the same tensor of the same head, so they take the same code
// path and meet the same barriers.
template <int D, int D0, int D1, int LAY, bool ROT>
__global__ __launch_bounds__(2 * kThreads, 1)
void k_qkv_proj_prologue2(QkvProjArgs a) {
  static_assert(D == 128, "one 128-channel head per prologue unit");
  constexpr int kRS = D / 2 + 1;
  constexpr int kStaged = kBlock * kRS * 4;            // staged fp16 tile (padded rows)
  constexpr int kPacked = kBlock * D * 2;              // packed fp16 tile
  constexpr int kBuf = kStaged + kPacked;
  constexpr int kT2 = 256 * kGRow;                     // one 256-row tile of a stage
  static_assert(kBuf >= 2 * kT2, "a stage fits in one buffer");
  // buffer h: stage h of the projection, then the staged tile of token block
  // 2i+h and the packed tile of the second (tensor, head); separate arrays,
  // so that the compiler sees that the next stage's loads never alias the
  // operand reads of the current one
  __shared__ __align__(16) uint8_t buf0[kBuf];
  __shared__ __align__(16) uint8_t buf1[kBuf];
  __shared__ float red[32];
  typedef __attribute__((address_space(3))) void* lds_ptr;

  // tile: each XCD works through groups of 32 tiles = 8 token-block pairs x
  // 4 pairs of (tensor, head) pairs
  const int H = a.p.H, NB = a.p.NB, N = a.p.N;
  const int TPB = NB / 2;                              // token-block pairs per batch entry
  const int L = blockIdx.x;
  const int S = (L / 256) * 8 + (L % 8);
  const int r = (L / 8) % 32;
  if (S >= a.SBT * a.SHT) return;
  const int tp = (S % a.SBT) * 8 + (r % 8);
  const int hp = (S / a.SBT) * 4 + (r / 8);
  if (tp >= a.B * TPB || hp >= 3 * H / 2) return;
  const int b = tp / TPB, blk0 = 2 * (tp % TPB), ht0 = 2 * hp;
  const int n00 = blk0 * kBlock;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;   // 8 waves
  const int col = lane & 31, hh = lane >> 5;
  const int wc = w & 3, wt = w >> 2;           // wave's 64 channels of 256, token block of the pair
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // stage loads: wave instruction i (0..3) fills the 1 KiB window 8i + w of a
  // 256-row tile, rows 8 (8i + w) + lane/8; rows 64 apart share the swizzle key
  const int lrow = 8 * w + lane / 8;
  const int lchunk = (lane % 8) ^ gswz(lrow);
  const size_t wrow_bytes = (size_t)a.C * 2;
  const uint8_t* wbase = (const uint8_t*)(a.w + (size_t)ht0 * D * a.C);
  const uint32_t woff = (uint32_t)(lrow * wrow_bytes) + 16 * lchunk;
  const uint8_t* xbase = (const uint8_t*)(a.x + (int64_t)b * a.x_batch + (int64_t)n00 * a.x_token);
  const int rmax = (N - n00 < 2 * kBlock ? N - n00 : 2 * kBlock) - 1;
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = lrow + 64 * i;
    xoff[i] = (uint32_t)((int64_t)(row < rmax ? row : rmax) * a.x_token * 2) + 16 * lchunk;
  }
  auto gload = [&](int it, uint8_t* slot) {
    uint32_t wo = woff, xo0 = xoff[0], xo1 = xoff[1], xo2 = xoff[2], xo3 = xoff[3];
    asm volatile("" : "+v"(wo), "+v"(xo0), "+v"(xo1), "+v"(xo2), "+v"(xo3));
    const uint32_t xo[4] = {xo0, xo1, xo2, xo3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* wb = wbase + (size_t)it * kGRow + (size_t)64 * i * wrow_bytes;
      const uint8_t* xb = xbase + (size_t)it * kGRow;
      asm volatile("" : "+s"(wb), "+s"(xb));
      __builtin_amdgcn_global_load_lds((const void*)(wb + wo),
                                       (lds_ptr)(slot + (8 * i + wu) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(xb + xo[i]),
                                       (lds_ptr)(slot + kT2 + (8 * i + wu) * 1024), 16, 0, 0);
    }
  };

  uint32_t xa = (64 * wc + col) * kGRow + 16 * (hh ^ gswz(64 * wc + col));
  uint32_t xb = kT2 + (128 * wt + col) * kGRow + 16 * (hh ^ gswz(128 * wt + col));
  asm volatile("" : "+v"(xa), "+v"(xb));
  v16f acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v16f{0.0f};
  const int kIters = a.C / kGK;

  // stage it from `cur`: request stage it+1 into `next` (last read in
  // iteration it-1, before the barrier), 32 MFMAs, wait, barrier
  auto step = [&](int it, const uint8_t* cur, uint8_t* next) {
    if (it + 1 < kIters) gload(it + 1, next);
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      v8h fa[2], fb[4];
#pragma unroll
      for (int m = 0; m < 2; ++m) fa[m] = *(const v8h*)(cur + ((xa + 32 * kGRow * m) ^ (32 * ks)));
#pragma unroll
      for (int m = 0; m < 4; ++m) fb[m] = *(const v8h*)(cur + ((xb + 32 * kGRow * m) ^ (32 * ks)));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  gload(0, buf0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll 1
  for (int it = 0; it < kIters; it += 2) {
    step(it, buf0, buf1);
    if (it + 1 < kIters) step(it + 1, buf1, buf0);
  }

  // epilogue 1: + bias, fp16; the first (tensor, head)'s channels (waves with
  // wc < 2) into the staged layout of buffer wt, the second's packed beside it
  // (the last barrier above has every stage read done)
  uint8_t* mybuf = wt == 0 ? buf0 : buf1;
  uint32_t* xs = (uint32_t*)mybuf;
  uint32_t* pk = (uint32_t*)(mybuf + kStaged);
  const int second = wc >> 1;
  const int htw = ht0 + second;
  const int nvalid = N - (n00 + kBlock * wt);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int tok = 32 * ni + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 64 * (wc & 1) + 32 * mi + 8 * g + 4 * hh;   // channel within the head
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[mi][ni][4 * g + e];
          if (a.bias) v[e] += h2f(a.bias[(size_t)htw * D + c0 + e]);
        }
        uint32_t p0 = (uint32_t)f2h(v[0]) | ((uint32_t)f2h(v[1]) << 16);
        uint32_t p1 = (uint32_t)f2h(v[2]) | ((uint32_t)f2h(v[3]) << 16);
        if (tok >= nvalid) p0 = p1 = 0u;
        if (second == 0) {
          xs[tok * kRS + c0 / 2] = p0;
          xs[tok * kRS + c0 / 2 + 1] = p1;
        } else {
          // packed row of 64 dwords, dword d at d ^ (tok & 63): conflict-free
          // writes down a column of tokens and reads along a row
          pk[tok * 64 + ((c0 / 2) ^ (tok & 63))] = p0;
          pk[tok * 64 + ((c0 / 2 + 1) ^ (tok & 63))] = p1;
        }
      }
    }
  __syncthreads();

  // epilogue 2: two rounds of prologue units, half wt on token block blk0+wt
  const size_t BH = (size_t)a.B * H, N_pad = (size_t)NB * kBlock;
  const int blk = blk0 + wt, n0 = blk * kBlock;
  float* myred = red + 16 * wt;
  auto unit = [&](int ht) {
    const int t = ht / H, bh = b * H + ht % H;
    if (a.qkv_out) store_tile_all<D>(a.qkv_out + ((size_t)t * BH + bh) * N_pad * D, n0, xs);
    if (a.p.fallback.test(bh)) {
      if (t < 2) {
        rope_fallback<D, D0, D1>(a.p, xs, n0);
        __syncthreads();
        store_tile_all<D>((t == 0 ? a.p.q_rope : a.p.k_rope) + (size_t)bh * N_pad * D, n0, xs);
      } else {
        store_vt_tiles<D>(xs, a.p.v_t + ((size_t)bh * N_pad + n0) * D);
      }
    } else if (t < 2) {
      quant_qk_tile<D, D0, D1, LAY, ROT>(a.p, xs, myred, t, blk, bh, [] {});
    } else {
      quant_v_tile<D, LAY>(a.p, xs, myred, blk, bh);
    }
  };
  unit(ht0);
  __syncthreads();
  // the second (tensor, head)'s tile of this half: packed -> staged layout
  for (int i = ltid(); i < kBlock * 64; i += kThreads) {
    const int tok = i >> 6, d = i & 63;
    xs[tok * kRS + d] = pk[tok * 64 + (d ^ (tok & 63))];
  }
  __syncthreads();
  unit(ht0 + 1);
}

template <int LAY>
static void launch_qkv_proj_l(bool rot, dim3 grid, const QkvProjArgs& a, hipStream_t st) {
  if (rot)
    hipLaunchKernelGGL((k_qkv_proj_prologue<128, 44, 42, LAY, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_qkv_proj_prologue<128, 44, 42, LAY, false>), grid, dim3(kThreads), 0, st, a);
}

template <int LAY>
static void launch_qkv_proj2_l(bool rot, dim3 grid, const QkvProjArgs& a, hipStream_t st) {
  if (rot)
    hipLaunchKernelGGL((k_qkv_proj_prologue2<128, 44, 42, LAY, true>), grid, dim3(2 * kThreads), 0,
                       st, a);
  else
    hipLaunchKernelGGL((k_qkv_proj_prologue2<128, 44, 42, LAY, false>), grid, dim3(2 * kThreads), 0,
                       st, a);
}

template <int LAY>
static void launch_qkv_proj_all(bool rot, const QkvProjArgs& a0, hipStream_t st) {
  const int H = a0.p.H, NB = a0.p.NB;
  if (H % 2 == 0 && NB >= 2) {
    // 256 x 256 tiles over the token-block pairs, then the 128 x 128 kernel
    // on the last block of each batch entry when NB is odd
    QkvProjArgs a = a0;
    a.SBT = (a.B * (NB / 2) + 7) / 8;
    a.SHT = (3 * H / 2 + 3) / 4;
    a.last_block_only = 0;
    launch_qkv_proj2_l<LAY>(rot, dim3((unsigned)(((a.SBT * a.SHT + 7) / 8) * 256)), a, st);
    if (NB % 2 == 1) {
      a.last_block_only = 1;
      launch_qkv_proj_l<LAY>(rot, dim3((unsigned)(a.B * 3 * H)), a, st);
    }
  } else {
    QkvProjArgs a = a0;
    a.SBT = (a.B * NB + 7) / 8;
    a.SHT = (3 * H + 7) / 8;
    a.last_block_only = 0;
    launch_qkv_proj_l<LAY>(rot, dim3((unsigned)(((a.SBT * a.SHT + 7) / 8) * 512)), a, st);
  }
}

hipError_t launch_qkv_proj(int D, int dt, int layout, bool rot, const QkvProjArgs& a,
                           hipStream_t st) {
  if (D != 128 || dt != 44) return hipErrorInvalidValue;
  if (layout == ROTATTN_LAYOUT_FP8)
    launch_qkv_proj_all<ROTATTN_LAYOUT_FP8>(rot, a, st);
  else if (layout == ROTATTN_LAYOUT_FP6)
    launch_qkv_proj_all<ROTATTN_LAYOUT_FP6>(rot, a, st);
  else
    launch_qkv_proj_all<ROTATTN_LAYOUT_PACKED>(rot, a, st);
  return hipGetLastError();
}

}  // namespace rotattn

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
}

hipError_t launch_rot_to_f64(const float* rt, const float* rh, const float* rw, int dt, int dh,
                             double* out, hipStream_t st) {
  hipLaunchKernelGGL(k_rot_to_f64, dim3(16), dim3(256), 0, st, rt, rh, rw, dt, dh, out);
  return hipGetLastError();
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide amax -> (inv, scale); every thread gets both.
__device__ __forceinline__ void block_scale(float local, float* red, float& inv, float& scale) {
  const int w = threadIdx.x >> 6;
  local = wave_max(local);
  if ((threadIdx.x & 63) == 0) red[w] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
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
// conversion to fp64 at each use is exact).  rot is [k][r] in fp64.
template <int DA>
__device__ __forceinline__ void load_rot_frags(const double* rot,
                                               float (&b)[Part<DA>::KS][Part<DA>::JB]) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int ks = 0; ks < Part<DA>::KS; ++ks)
#pragma unroll
    for (int jb = 0; jb < Part<DA>::JB; ++jb) {
      const int k = 4 * ks + (l >> 4), j = 16 * jb + (l & 15);
      // unconditional (clamped) loads: all of them in flight at once
      const float r = (float)rot[min(k, DA - 1) * DA + min(j, DA - 1)];
      b[ks][jb] = (k < DA && j < DA) ? r : 0.0f;
    }
}

// Position of token n (< N) on RoPE axis `axis`: t = n / (Hg Wg),
// h = (n / Wg) mod Hg, w = n mod Wg.  Padding tokens (n >= N) have zero rows;
// any valid table row will do for them.
__device__ __forceinline__ int axis_pos(int n, int N, int axis, int HW, int gh, int gw) {
  return n < N ? (axis == 0 ? n / HW : (axis == 1 ? (n / gw) % gh : n % gw)) : 0;
}

// The RoPE'd value of channel c (< DA) of one partition for one token: the
// token's staged fp16 row xrow (one dword per channel pair, partition start),
// its table rows start at element trow of cos_a and sin_a.  Even channel:
// fl(x0 c) - fl(x1 s); odd channel: fl(x0 s) + fl(x1 c).  Operands are
// selected instead of branching (negation is exact).  Channels >= DA (MFMA
// zero padding) read a clamped pair.
template <int DA>
__device__ __forceinline__ float rope_channel(const uint32_t* xrow, const float* cos_a,
                                              const float* sin_a, int trow, int c) {
  const int jp = (c >> 1) < DA / 2 ? (c >> 1) : DA / 2 - 1;
  const uint32_t pr = xrow[jp];
  const float x0 = h2f((uint16_t)(pr & 0xffffu));
  const float x1 = h2f((uint16_t)(pr >> 16));
  const float cs = cos_a[trow + jp], sn = sin_a[trow + jp];
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
__device__ __forceinline__ float rotate_part(const uint32_t* xs, const float* cos_a,
                                             const float* sin_a,
                                             float (&b)[Part<DA>::KS][Part<DA>::JB], int off,
                                             int tok0, int n0, int N, int axis, int HW, int gh,
                                             int gw, float (&z)[TB][Part<DA>::JB][4]) {
  constexpr int KS = Part<DA>::KS, JB = Part<DA>::JB;
  const int l = threadIdx.x & 63;
  float amax = 0.0f;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    // the fp32 fragments are marked as changing here so that their fp64
    // conversions stay next to the MFMAs instead of being hoisted into
    // 2 x KS x JB live registers
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) asm volatile("" : "+v"(b[ks][jb]));
    const int i = tok0 + 16 * tb + (l & 15);   // this lane's A row (token in the block)
    const int pos = axis_pos(n0 + i, N, axis, HW, gh, gw);
    const uint32_t* xrow = xs + i * kRS + off / 2;
    const int trow = pos * (DA / 2);
    // RoPE'd A fragments of this token group, then the MFMA chain over k
    double av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 4 * ks + (l >> 4);                      // channel in the partition
      const float y = rope_channel<DA>(xrow, cos_a, sin_a, trow, c);
      av[ks] = c < DA ? (double)y : 0.0;
    }
    v4d acc[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[jb] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
        acc[jb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ks], (double)b[ks][jb], acc[jb], 0, 0, 0);
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[tb][jb][r] = (float)acc[jb][r];
        amax = fmaxf(amax, fabsf(z[tb][jb][r]));
      }
  }
  return amax;
}

// RoPE only, for rotations merged into the RoPE tables (per-pair 2x2
// rotations commute with RoPE, so R RoPE(p) = RoPE with phase offsets):
// z = y = RoPE(x) exactly as the rotating path computes its A fragments, kept
// in that layout (token tok0 + 16 tb + l%16, channel 4 ks + l/16).  Returns
// the lane's max |z|.
template <int DA, int TB, int kRS>
__device__ __forceinline__ float rope_part_a(const uint32_t* xs, const float* cos_a,
                                             const float* sin_a, int off, int tok0, int n0, int N,
                                             int axis, int HW, int gh, int gw,
                                             float (&z)[TB][Part<DA>::KS]) {
  constexpr int KS = Part<DA>::KS;
  const int l = threadIdx.x & 63;
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
      const float y = rope_channel<DA>(xrow, cos_a, sin_a, trow, c);
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
  const int l = threadIdx.x & 63;
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
  const int l = threadIdx.x & 63;
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
  const int n = threadIdx.x & (kBlock - 1), h = threadIdx.x / kBlock;
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
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  for (int i = threadIdx.x; i < kBlock * kChunks; i += kThreads) {
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
  for (int item = threadIdx.x; item < 2 * D * 8; item += kThreads) {
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
  for (int i = threadIdx.x; i < kBlock * kDw; i += kThreads) {
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
  for (int i = threadIdx.x; i < kBlock * kDw; i += kThreads) {
    const int n = i / kDw, g = i % kDw;
    *(uint32_t*)(dst + (size_t)n * D + 4 * g) = *(const uint32_t*)(codes + n * kCodeStride + 4 * g);
  }
}

// FP8 layout: V code bytes (LDS, [channel][token]) -> V^T block [D][128], each
// 64-key half in the P.V operand order (byte 32h + j of a half holds key
// 32(j/16) + 8((j%16)/4) + 4h + j%4).  Dwords move whole: j%4 is the byte.
template <int D>
__device__ __forceinline__ void store_v_codes_f8(const int8_t* codesT, uint8_t* dst) {
  for (int i = threadIdx.x; i < D * 32; i += kThreads) {
    const int d = i / 32, q = i % 32;                 // output dword q of row d
    const int c = q / 16, h = (q / 8) & 1, j = 4 * (q & 7);
    const int key = 64 * c + 32 * (j / 16) + 8 * ((j % 16) / 4) + 4 * h;
    *(uint32_t*)(dst + (size_t)d * 128 + 4 * q) = *(const uint32_t*)(codesT + d * kCodeStride + key);
  }
}

// V codes (LDS, [channel][token]) -> packed V^T block [D][64] in global memory.
template <int D>
__device__ __forceinline__ void store_v_codes(const int8_t* codesT, uint8_t* dst) {
  for (int i = threadIdx.x; i < D * 16; i += kThreads) {
    const int d = i / 16, g = i % 16;
    const uint32_t lo = *(const uint32_t*)(codesT + d * kCodeStride + 8 * g);
    const uint32_t hi = *(const uint32_t*)(codesT + d * kCodeStride + 8 * g + 4);
    *(uint32_t*)(dst + (size_t)d * 64 + 4 * g) = pack_nibbles(lo, hi);
  }
}

// A head that is not a fallback head.  Wave w owns tokens 32w..32w+31 of the
// block in every partition: per tensor, RoPE + rotation on the MFMA (or RoPE
// alone), block amax, codes into the LDS buffer that held the tensor's rows,
// coalesced store; then V: block amax and codes, stored transposed.
template <int D, int D0, int D1, bool F8, bool ROT>
__device__ __forceinline__ void prologue_qk(const PrologueArgs& a, uint32_t* stage_q,
                                            uint32_t* stage_k, float* red, int blk, int bh) {
  constexpr int kRS = D / 2 + 1;
  constexpr int TB = kBlock / 16 / (kThreads / 64);   // 16-token groups per wave
  const int w = threadIdx.x >> 6;
  const int tok0 = 16 * TB * w;
  const int n0 = blk * kBlock;
  const int HW = a.grid_h * a.grid_w;
  const int64_t head_in = a.in.head_offset(bh, a.H);
  const size_t pad_row = ((size_t)bh * a.NB + blk) * kBlock;   // first code row of this block

  load_tile<D>(a.q + head_in, a.in.token, n0, a.N, stage_q);
  load_tile<D>(a.k + head_in, a.in.token, n0, a.N, stage_k);
  wait_tiles();
  __syncthreads();

  // one tensor (s = 0: Q, 1: K), inlined twice: straight-line code, so
  // nothing is hoisted across the two tensors and kept live
  auto tensor = [&](int s) {
    uint32_t* xs = s == 0 ? stage_q : stage_k;
    int8_t* codes = (int8_t*)xs;
    float inv, scale;
    // the table reads are the same for Q and K; an opaque zero offset per
    // tensor keeps the compiler from loading them once and holding them in
    // registers across both tensors
    int zero = 0;
    asm volatile("" : "+s"(zero));
    const float *cos_t = a.cos_t + zero, *sin_t = a.sin_t + zero, *cos_h = a.cos_h + zero;
    const float *sin_h = a.sin_h + zero, *cos_w = a.cos_w + zero, *sin_w = a.sin_w + zero;
    // every wave is past its last read of xs once the reduction's barriers are
    // passed: the buffer takes the codes next
    if (ROT) {
      // R_a^T of each partition as B fragments, loaded (from cache) just before
      // its use; rotation matrices in fp64 [k][r]: t at 0, h at D0^2, w at
      // D0^2 + D1^2
      float z0[TB][Part<D0>::JB][4], z1[TB][Part<D1>::JB][4], z2[TB][Part<D1>::JB][4];
      float amax;
      {
        float b[Part<D0>::KS][Part<D0>::JB];
        const double* rp = a.rot64 + zero;   // read again per tensor, not held
        load_rot_frags<D0>(rp, b);
        amax = rotate_part<D0, TB, kRS>(xs, cos_t, sin_t, b, 0, tok0, n0, a.N, 0, HW, a.grid_h,
                                        a.grid_w, z0);
      }
      {
        float b[Part<D1>::KS][Part<D1>::JB];
        const double* rp = a.rot64 + D0 * D0 + zero;
        load_rot_frags<D1>(rp, b);
        amax = fmaxf(amax, rotate_part<D1, TB, kRS>(xs, cos_h, sin_h, b, D0, tok0, n0, a.N, 1,
                                                    HW, a.grid_h, a.grid_w, z1));
      }
      {
        float b[Part<D1>::KS][Part<D1>::JB];
        const double* rp = a.rot64 + D0 * D0 + D1 * D1 + zero;
        load_rot_frags<D1>(rp, b);
        amax = fmaxf(amax, rotate_part<D1, TB, kRS>(xs, cos_w, sin_w, b, D0 + D1, tok0, n0,
                                                    a.N, 2, HW, a.grid_h, a.grid_w, z2));
      }
      block_scale(amax, red, inv, scale);
      // K pass, past the reduction's barriers: every wave is done with the Q
      // codes in stage_q and has issued its last table load, so V's rows can
      // stream in while K is quantized and stored
      if (s == 1) load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage_q);
      quant_part<D0, TB, F8>(z0, inv, 0, tok0, codes);
      quant_part<D1, TB, F8>(z1, inv, D0, tok0, codes);
      quant_part<D1, TB, F8>(z2, inv, D0 + D1, tok0, codes);
    } else {
      float z0[TB][Part<D0>::KS], z1[TB][Part<D1>::KS], z2[TB][Part<D1>::KS];
      float amax = rope_part_a<D0, TB, kRS>(xs, cos_t, sin_t, 0, tok0, n0, a.N, 0, HW,
                                            a.grid_h, a.grid_w, z0);
      amax = fmaxf(amax, rope_part_a<D1, TB, kRS>(xs, cos_h, sin_h, D0, tok0, n0, a.N, 1, HW,
                                                  a.grid_h, a.grid_w, z1));
      amax = fmaxf(amax, rope_part_a<D1, TB, kRS>(xs, cos_w, sin_w, D0 + D1, tok0, n0, a.N,
                                                  2, HW, a.grid_h, a.grid_w, z2));
      block_scale(amax, red, inv, scale);
      if (s == 1) load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage_q);
      quant_part_a<D0, TB, F8>(z0, inv, 0, tok0, codes);
      quant_part_a<D1, TB, F8>(z1, inv, D0, tok0, codes);
      quant_part_a<D1, TB, F8>(z2, inv, D0 + D1, tok0, codes);
    }
    __syncthreads();
    if (F8)
      store_qk_codes_f8<D>(codes, (s == 0 ? a.q4 : a.k4) + pad_row * D);
    else
      store_qk_codes<D>(codes, (s == 0 ? a.q4 : a.k4) + pad_row * (D / 2));
    if (threadIdx.x == 0) {
      if (s == 0)
        a.q_scale_l2[(size_t)bh * a.NB + blk] = scale * a.kappa;
      else
        a.k_scale[(size_t)bh * a.NB + blk] = scale;
    }
  };
  tensor(0);
  tensor(1);
  __syncthreads();

  // V: staged in the Q buffer (requested during the K pass), codes in place
  wait_tiles();
  __syncthreads();
  int8_t* codes = (int8_t*)stage_q;
  float scale;
  v_codes<D, F8>(stage_q, red, codes, scale);
  __syncthreads();
  if (F8)
    store_v_codes_f8<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 128);
  else
    store_v_codes<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 64);
  if (threadIdx.x == 0) a.v_scale[(size_t)bh * a.NB + blk] = scale;
}

// Fallback head, RoPE of one staged tensor in place: thread (token n, half h)
// applies RoPE to partition t (h = 0) or partitions h and w (h = 1) of its
// token's row in fp32 and writes the fp16 pairs back once every thread has
// read its row.
template <int D, int D0, int D1>
__device__ __forceinline__ void rope_fallback(const PrologueArgs& a, uint32_t* xs, int n0) {
  constexpr int kRS = D / 2 + 1;
  constexpr int NY = D0 > 2 * D1 ? D0 : 2 * D1;
  const int n = threadIdx.x & (kBlock - 1);
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x / kBlock);
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

// One work-group per (128-token block, head), 4 waves (one per SIMD): two
// work-groups share a CU (LDS), so one group's MFMA phase overlaps the other's
// memory phases.
template <int D, int D0, int D1, bool F8, bool ROT>
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
    prologue_qk<D, D0, D1, F8, ROT>(a, stage_q, stage_k, red, blk, bh);
}

template <int D, int D0, int D1>
static void launch_prologue_t(bool f8, bool rot, dim3 grid, const PrologueArgs& a, hipStream_t st) {
  if (f8) {
    if (rot)
      hipLaunchKernelGGL((k_prologue<D, D0, D1, true, true>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((k_prologue<D, D0, D1, true, false>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (rot)
      hipLaunchKernelGGL((k_prologue<D, D0, D1, false, true>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((k_prologue<D, D0, D1, false, false>), grid, dim3(kThreads), 0, st, a);
  }
}

hipError_t launch_prologue(int D, int dt, int BH, bool f8, bool rot, const PrologueArgs& a,
                           hipStream_t st) {
  dim3 grid(a.NB, BH);
  if (D == 128 && dt == 44)
    launch_prologue_t<128, 44, 42>(f8, rot, grid, a, st);
  else if (D == 64 && dt == 24)
    launch_prologue_t<64, 24, 20>(f8, rot, grid, a, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rotattn

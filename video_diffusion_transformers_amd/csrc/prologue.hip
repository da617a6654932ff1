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
// One work-group per (128-token block, head); 384 threads = 6 waves.
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
// k reproduce the sequential fp64 sum exactly.  Wave 2a + h owns partition a
// and tokens 64h..64h+63: R_a^T sits in its registers as B fragments, and the A
// fragments are RoPE'd on the fly from the staged fp16 rows.
#include "rotattn_internal.h"

namespace rotattn {

constexpr int kThreads = 384;
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

__device__ __forceinline__ int quant(float z, float inv) {
  return (int)fminf(fmaxf(rintf(z * inv), -7.0f), 7.0f);
}

// FP8 E4M3 bits of an integer code in [-7, 7] (exact: 1 = 0x38, 2 = 0x40,
// 3 = 0x44, ..., 7 = 0x4E; sign in bit 7).
__device__ __forceinline__ uint32_t e4m3_of(int c) {
  const uint64_t lut = 0x4E4C4A4844403800ull;
  const uint32_t mag = (uint32_t)(c < 0 ? -c : c);
  return (uint32_t)((lut >> (8 * mag)) & 0xFFu) | (c < 0 ? 0x80u : 0u);
}

// The byte stored for a code: int8 for the packed layout, E4M3 for FP8.
template <bool F8>
__device__ __forceinline__ int8_t code_byte(int c) {
  return F8 ? (int8_t)e4m3_of(c) : (int8_t)c;
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

// RoPE + rotation of one tensor over this wave's partition (width DA at channel
// offset off) and 64 tokens (tok0..tok0+63 of the block): z in the MFMA output
// layout (token row tok0 + 16 tb + l/16 + 4 r, channel 16 jb + l%16), returns
// the lane's max |z|.  xs: staged fp16 rows of the tensor (kRS dwords per row).
template <int DA, int kRS>
__device__ __forceinline__ float rotate_tensor(const uint32_t* xs, const float* cos_a,
                                               const float* sin_a,
                                               float (&b)[Part<DA>::KS][Part<DA>::JB], int off,
                                               int tok0, int n0, int N, int axis, int HW, int gh,
                                               int gw, float (&z)[4][Part<DA>::JB][4]) {
  constexpr int KS = Part<DA>::KS, JB = Part<DA>::JB;
  const int l = threadIdx.x & 63;
  float amax = 0.0f;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    // the fp32 fragments are marked as changing here so that their fp64
    // conversions stay next to the MFMAs instead of being hoisted into
    // 2 x KS x JB live registers
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) asm volatile("" : "+v"(b[ks][jb]));
    const int i = tok0 + 16 * tb + (l & 15);   // this lane's A row (token in the block)
    const int n = n0 + i;
    // padding tokens have zero rows; any valid table row will do
    const int pos = n < N ? (axis == 0 ? n / HW : (axis == 1 ? (n / gw) % gh : n % gw)) : 0;
    const uint32_t* xrow = xs + i * kRS + off / 2;
    const float* crow = cos_a + pos * (DA / 2);
    const float* srow = sin_a + pos * (DA / 2);
    // RoPE'd A fragments of this token block, then the MFMA chain over k
    double av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 4 * ks + (l >> 4);                      // channel in the partition
      const int jp = (c >> 1) < DA / 2 ? (c >> 1) : DA / 2 - 1;   // pair (clamped on padding)
      const uint32_t pr = xrow[jp];
      const float x0 = h2f((uint16_t)(pr & 0xffffu));
      const float x1 = h2f((uint16_t)(pr >> 16));
      const float cs = crow[jp], sn = srow[jp];
      // even channel: fl(x0 c) - fl(x1 s); odd: fl(x0 s) + fl(x1 c); operands
      // are selected instead of branching (negation is exact)
      const bool odd = (c & 1) != 0;
      const float p0 = x0 * (odd ? sn : cs);
      const float p1 = x1 * (odd ? cs : sn);
      const float y = p0 + (odd ? p1 : -p1);
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
template <int DA, int kRS>
__device__ __forceinline__ float rope_tensor(const uint32_t* xs, const float* cos_a,
                                             const float* sin_a, int off, int tok0, int n0, int N,
                                             int axis, int HW, int gh, int gw,
                                             float (&z)[4][Part<DA>::KS]) {
  constexpr int KS = Part<DA>::KS;
  const int l = threadIdx.x & 63;
  float amax = 0.0f;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int i = tok0 + 16 * tb + (l & 15);
    const int n = n0 + i;
    const int pos = n < N ? (axis == 0 ? n / HW : (axis == 1 ? (n / gw) % gh : n % gw)) : 0;
    const uint32_t* xrow = xs + i * kRS + off / 2;
    const float* crow = cos_a + pos * (DA / 2);
    const float* srow = sin_a + pos * (DA / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 4 * ks + (l >> 4);
      const int jp = (c >> 1) < DA / 2 ? (c >> 1) : DA / 2 - 1;
      const uint32_t pr = xrow[jp];
      const float x0 = h2f((uint16_t)(pr & 0xffffu));
      const float x1 = h2f((uint16_t)(pr >> 16));
      const float cs = crow[jp], sn = srow[jp];
      const bool odd = (c & 1) != 0;
      const float p0 = x0 * (odd ? sn : cs);
      const float p1 = x1 * (odd ? cs : sn);
      const float y = p0 + (odd ? p1 : -p1);
      z[tb][ks] = c < DA ? y : 0.0f;
      amax = fmaxf(amax, fabsf(z[tb][ks]));
    }
  }
  return amax;
}

// Codes of rope_tensor's z (A layout) into the LDS code buffer.
template <int DA, bool F8>
__device__ __forceinline__ void quant_tensor_a(const float (&z)[4][Part<DA>::KS], float inv,
                                               int off, int tok0, int8_t* codes) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int ks = 0; ks < Part<DA>::KS; ++ks) {
      const int c = 4 * ks + (l >> 4);
      if (c < DA)
        codes[(tok0 + 16 * tb + (l & 15)) * kCodeStride + off + c] = code_byte<F8>(quant(z[tb][ks], inv));
    }
}

// Codes of one tensor's z (MFMA output layout) into the LDS code buffer
// ([token][channel], kCodeStride bytes per row).
template <int DA, bool F8>
__device__ __forceinline__ void quant_tensor(const float (&z)[4][Part<DA>::JB][4], float inv,
                                             int off, int tok0, int8_t* codes) {
  constexpr int JBX = Part<DA>::JB;
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int jb = 0; jb < JBX; ++jb) {
      const int j = 16 * jb + (l & 15);
      if (j < DA) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = tok0 + 16 * tb + (l >> 4) + 4 * r;
          codes[row * kCodeStride + off + j] = code_byte<F8>(quant(z[tb][jb][r], inv));
        }
      }
    }
}

// Fallback head: RoPE'd fp16 pairs written back over the staged row (the
// caller stores the tile with coalesced writes).
template <int DA>
__device__ __forceinline__ void rope_only_part(uint32_t* xrow, const float* cos_a,
                                               const float* sin_a, int pos, int off) {
  float y[DA];
  rope_part<DA>(xrow, cos_a, sin_a, pos, off, y);
  __syncthreads();   // every lane has read its inputs before any row is overwritten
#pragma unroll
  for (int j = 0; j < DA / 2; ++j)
    xrow[off / 2 + j] = (uint32_t)f2h(y[2 * j]) | ((uint32_t)f2h(y[2 * j + 1]) << 16);
}

template <int DA, bool F8>
__device__ __forceinline__ void v_part(const uint32_t* xrow, int off, float* red,
                                       int8_t* codesT, int nl, float& scale_out) {
  float x[DA];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < DA / 2; ++j) {
    const uint32_t pr = xrow[off / 2 + j];
    x[2 * j] = h2f((uint16_t)(pr & 0xffffu));
    x[2 * j + 1] = h2f((uint16_t)(pr >> 16));
    amax = fmaxf(amax, fmaxf(fabsf(x[2 * j]), fabsf(x[2 * j + 1])));
  }
  float inv, scale;
  block_scale(amax, red, inv, scale);
#pragma unroll
  for (int r = 0; r < DA; ++r) codesT[(off + r) * kCodeStride + nl] = code_byte<F8>(quant(x[r], inv));
  scale_out = scale;
}

// Coalesced load of a block's fp16 rows [128][D] into LDS rows of D/2 + 1
// dwords (the odd stride keeps the per-token reads conflict-free); rows past
// N are zero.
// Stage 128 fp16 rows (tokens n0..n0+127 of one head, row_stride elements
// apart) into xs, kRS dwords per row, zero rows for tokens >= N.  Each wave
// instruction moves one row straight from memory into LDS (global_load_lds,
// lane L -> dword L of the row): no registers, no waits here.  The caller
// waits with wait_tiles() before the barrier that publishes the rows.
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

// A head that is not a fallback head, as seen by one wave (partition of width
// DA at channel offset off, RoPE axis `axis`): per tensor, RoPE + rotation on
// the MFMA, block amax, codes into the LDS buffer that held the tensor's rows,
// coalesced store; then V: block amax and codes, stored transposed.  Every
// wave runs the same sequence of barriers whatever its partition.
template <int D, int DA, bool F8, bool ROT>
__device__ __forceinline__ void prologue_qk(const PrologueArgs& a, uint32_t* stage_q,
                                            uint32_t* stage_k, float* red, int blk, int bh,
                                            int off, int axis, const float* cos_a,
                                            const float* sin_a, const double* rot) {
  constexpr int kRS = D / 2 + 1;
  const int w = threadIdx.x >> 6;
  const int tok0 = (w & 1) * 64;
  const int n0 = blk * kBlock;
  const int HW = a.grid_h * a.grid_w;
  const int64_t head_in = a.in.head_offset(bh, a.H);
  const size_t pad_row = ((size_t)bh * a.NB + blk) * kBlock;   // first code row of this block

  load_tile<D>(a.q + head_in, a.in.token, n0, a.N, stage_q);
  load_tile<D>(a.k + head_in, a.in.token, n0, a.N, stage_k);
  float b[Part<DA>::KS][Part<DA>::JB];   // R_a^T of this wave's partition
  if (ROT) load_rot_frags<DA>(rot, b);
  wait_tiles();
  __syncthreads();

#pragma unroll 1
  for (int s = 0; s < 2; ++s) {
    uint32_t* xs = s == 0 ? stage_q : stage_k;
    int8_t* codes = (int8_t*)xs;
    float inv, scale;
    // every wave is past its last read of xs once the reduction's barriers are
    // passed: the buffer takes the codes next
    if (ROT) {
      float z[4][Part<DA>::JB][4];
      const float amax = rotate_tensor<DA, kRS>(xs, cos_a, sin_a, b, off, tok0, n0, a.N, axis, HW,
                                                a.grid_h, a.grid_w, z);
      block_scale(amax, red, inv, scale);
      quant_tensor<DA, F8>(z, inv, off, tok0, codes);
    } else {
      float z[4][Part<DA>::KS];
      const float amax = rope_tensor<DA, kRS>(xs, cos_a, sin_a, off, tok0, n0, a.N, axis, HW,
                                              a.grid_h, a.grid_w, z);
      block_scale(amax, red, inv, scale);
      quant_tensor_a<DA, F8>(z, inv, off, tok0, codes);
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
  }
  __syncthreads();

  // V: staged in the Q buffer, codes (channel rows) in the K buffer
  const int nl = tok0 + (threadIdx.x & 63);
  load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage_q);
  wait_tiles();
  __syncthreads();
  int8_t* codes = (int8_t*)stage_k;
  float scale;
  v_part<DA, F8>(stage_q + nl * kRS, off, red, codes, nl, scale);
  __syncthreads();
  if (F8)
    store_v_codes_f8<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 128);
  else
    store_v_codes<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 64);
  if (threadIdx.x == 0) a.v_scale[(size_t)bh * a.NB + blk] = scale;
}

// Fallback head: RoPE'd fp16 Q and K into the padded q_rope/k_rope rows, one
// token per lane, wave pair a on partition a; then V^T tiles for the fp16
// attention.
template <int D, int D0, int D1>
__device__ __forceinline__ void prologue_fallback(const PrologueArgs& a, uint32_t* stage, int blk,
                                                  int bh) {
  constexpr int kRS = D / 2 + 1;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int part = __builtin_amdgcn_readfirstlane(w >> 1);
  const int nl = (w & 1) * 64 + lane;
  const int n0 = blk * kBlock;
  const int n = n0 + nl;
  const int HW = a.grid_h * a.grid_w;
  const int pos = part == 0 ? n / HW : (part == 1 ? (n / a.grid_w) % a.grid_h : n % a.grid_w);
  const int off = part == 0 ? 0 : (part == 1 ? D0 : D0 + D1);
  const float* cos_a = part == 0 ? a.cos_t : (part == 1 ? a.cos_h : a.cos_w);
  const float* sin_a = part == 0 ? a.sin_t : (part == 1 ? a.sin_h : a.sin_w);
  const int64_t head_in = a.in.head_offset(bh, a.H);
  const size_t head_pad = (size_t)bh * a.NB * kBlock;
  uint32_t* xrow = stage + nl * kRS;
  // tables are read for every lane; clamp the position of a padding token
  const int pos_c = n < a.N ? pos : 0;
#pragma unroll 1
  for (int s = 0; s < 2; ++s) {
    load_tile<D>((s == 0 ? a.q : a.k) + head_in, a.in.token, n0, a.N, stage);
    wait_tiles();
    __syncthreads();
    if (part == 0)
      rope_only_part<D0>(xrow, cos_a, sin_a, pos_c, off);
    else
      rope_only_part<D1>(xrow, cos_a, sin_a, pos_c, off);
    __syncthreads();
    store_tile_all<D>((s == 0 ? a.q_rope : a.k_rope) + head_pad * D, n0, stage);
    __syncthreads();
  }
  load_tile<D>(a.v + head_in, a.in.token, n0, a.N, stage);
  wait_tiles();
  __syncthreads();
  store_vt_tiles<D>(stage, a.v_t + (head_pad + n0) * D);
}

// 3 waves per SIMD: two 6-wave work-groups per CU, so that one group's MFMA
// phase overlaps the other's memory phases.
template <int D, int D0, int D1, bool F8, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void k_prologue(PrologueArgs a) {
  static_assert(D0 + 2 * D1 == D, "split must be (D0, D1, D1)");
  constexpr int kRS = D / 2 + 1;   // staged fp16 row, in dwords
  static_assert(kBlock * kCodeStride <= kBlock * kRS * 4, "codes fit in a staging buffer");
  static_assert(D * kCodeStride <= kBlock * kRS * 4, "transposed codes fit in a staging buffer");
  // two buffers of 128 staged fp16 rows (Q and K; later V and the codes)
  __shared__ __align__(16) uint32_t stage_q[kBlock * kRS];
  __shared__ __align__(16) uint32_t stage_k[kBlock * kRS];
  __shared__ float red[16];
  const int blk = blockIdx.x, bh = blockIdx.y;
  if (a.fallback.test(bh)) {
    prologue_fallback<D, D0, D1>(a, stage_q, blk, bh);
    return;
  }
  // wave pair 2a, 2a+1 on partition a; rotation matrices in fp64 [k][r]:
  // t at 0, h at D0^2, w at D0^2 + D1^2
  const int part = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) >> 1);
  if (part == 0)
    prologue_qk<D, D0, F8, ROT>(a, stage_q, stage_k, red, blk, bh, 0, 0, a.cos_t, a.sin_t, a.rot64);
  else if (part == 1)
    prologue_qk<D, D1, F8, ROT>(a, stage_q, stage_k, red, blk, bh, D0, 1, a.cos_h, a.sin_h,
                                a.rot64 + D0 * D0);
  else
    prologue_qk<D, D1, F8, ROT>(a, stage_q, stage_k, red, blk, bh, D0 + D1, 2, a.cos_w, a.sin_w,
                                a.rot64 + D0 * D0 + D1 * D1);
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

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
// One work-group per (128-token block, head); 384 threads = 6 waves; waves
// 2a, 2a+1 own RoPE partition a (t, h, w) for tokens 0-63 / 64-127 of the
// block, one token per lane.  Arithmetic (bit-exact by construction; this
// file is built with -ffp-contract=off):
//   RoPE   y0 = fl(fl(x0*c) - fl(x1*s)), y1 = fl(fl(x0*s) + fl(x1*c))   fp32
//   rotate z_r = fl32(sum_k R[r][k]*y_k): v_fma_f64 chain, k ascending (the
//          fp32 x fp32 products are exact in fp64), one rounding to fp32
//   INT4   per block: amax over the 128 tokens x D channels, inv = fl(7/amax),
//          scale = fl(amax/7), code = clamp(rne(fl(z*inv)), -7, 7)
// The rotation matrices are read as fp64 through the scalar unit (uniform
// addresses), so every MAC is one v_fma_f64 with an SGPR operand.
#include "rotattn_internal.h"

namespace rotattn {

__global__ void k_rot_to_f64(const float* rt, const float* rh, const float* rw, int dt, int dh,
                             int dw, double* out) {
  const int a = blockIdx.x;
  const float* src = a == 0 ? rt : (a == 1 ? rh : rw);
  const int d = a == 0 ? dt : (a == 1 ? dh : dw);
  for (int i = threadIdx.x; i < d * d; i += blockDim.x) out[a * 4096 + i] = (double)src[i];
}

hipError_t launch_rot_to_f64(const float* rt, const float* rh, const float* rw, int dt, int dh,
                             int dw, double* out, hipStream_t st) {
  hipLaunchKernelGGL(k_rot_to_f64, dim3(3), dim3(256), 0, st, rt, rh, rw, dt, dh, dw, out);
  return hipGetLastError();
}

constexpr int kThreads = 384;
constexpr int kCodeStride = 132;   // bytes per row of the int8 code buffers (33 dwords: no bank conflicts)

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// RoPE of this lane's token over one partition of width DA at channel offset
// off: y[0..DA) in fp32.
template <int DA>
__device__ __forceinline__ void rope_part(const uint16_t* row, bool valid, const float* cos_a,
                                          const float* sin_a, int pos, int off, float (&y)[DA]) {
#pragma unroll
  for (int j = 0; j < DA / 2; ++j) {
    uint32_t pr = valid ? *(const uint32_t*)(row + off + 2 * j) : 0u;
    const float x0 = h2f((uint16_t)(pr & 0xffffu));
    const float x1 = h2f((uint16_t)(pr >> 16));
    const float c = cos_a[pos * (DA / 2) + j];
    const float s = sin_a[pos * (DA / 2) + j];
    y[2 * j] = x0 * c - x1 * s;
    y[2 * j + 1] = x0 * s + x1 * c;
  }
}

// z = R y over one partition: fp64 accumulation, k ascending, one rounding.
template <int DA>
__device__ __forceinline__ void rotate_part(const float (&y)[DA], const double* __restrict__ R,
                                            float (&z)[DA]) {
  double yd[DA];
#pragma unroll
  for (int k = 0; k < DA; ++k) yd[k] = (double)y[k];
#pragma unroll
  for (int r = 0; r < DA; ++r) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < DA; ++k) acc = __builtin_fma(R[r * DA + k], yd[k], acc);
    z[r] = (float)acc;
  }
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

// One tensor (Q or K) of one partition for this lane's token: RoPE, rotation,
// block scale, codes into the LDS code buffer (row = token, padded stride).
template <int DA>
__device__ __forceinline__ void qk_part(const uint16_t* row, bool valid, const float* cos_a,
                                        const float* sin_a, int pos, int off, const double* R,
                                        float* red, int8_t* codes, int nl, float& scale_out) {
  float y[DA], z[DA];
  rope_part<DA>(row, valid, cos_a, sin_a, pos, off, y);
  rotate_part<DA>(y, R, z);
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < DA; ++r) amax = fmaxf(amax, fabsf(z[r]));
  float inv, scale;
  block_scale(amax, red, inv, scale);
#pragma unroll
  for (int r = 0; r < DA; ++r) codes[nl * kCodeStride + off + r] = (int8_t)quant(z[r], inv);
  scale_out = scale;
}

template <int DA>
__device__ __forceinline__ void rope_only_part(const uint16_t* row, bool valid, const float* cos_a,
                                               const float* sin_a, int pos, int off,
                                               uint16_t* out_row) {
  float y[DA];
  rope_part<DA>(row, valid, cos_a, sin_a, pos, off, y);
  if (!valid) return;
#pragma unroll
  for (int j = 0; j < DA / 2; ++j) {
    const uint32_t pr = (uint32_t)f2h(y[2 * j]) | ((uint32_t)f2h(y[2 * j + 1]) << 16);
    *(uint32_t*)(out_row + off + 2 * j) = pr;
  }
}

template <int DA>
__device__ __forceinline__ void v_part(const uint16_t* row, bool valid, int off, float* red,
                                       int8_t* codesT, int nl, float& scale_out) {
  float x[DA];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < DA / 2; ++j) {
    uint32_t pr = valid ? *(const uint32_t*)(row + off + 2 * j) : 0u;
    x[2 * j] = h2f((uint16_t)(pr & 0xffffu));
    x[2 * j + 1] = h2f((uint16_t)(pr >> 16));
    amax = fmaxf(amax, fmaxf(fabsf(x[2 * j]), fabsf(x[2 * j + 1])));
  }
  float inv, scale;
  block_scale(amax, red, inv, scale);
#pragma unroll
  for (int r = 0; r < DA; ++r) codesT[(off + r) * kCodeStride + nl] = (int8_t)quant(x[r], inv);
  scale_out = scale;
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

template <int D, int D0, int D1>
__global__ __launch_bounds__(kThreads) void k_prologue(PrologueArgs a) {
  static_assert(D0 + 2 * D1 == D, "split must be (D0, D1, D1)");
  __shared__ __align__(16) int8_t codes[kBlock * kCodeStride];   // 128 token rows, or D <= 128 channel rows
  __shared__ float red[16];

  const int blk = blockIdx.x, bh = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // wave-uniform: lets the rotation matrices and tables go through the scalar unit
  const int part = __builtin_amdgcn_readfirstlane(w >> 1);
  const int nl = (w & 1) * 64 + lane;
  const int n = blk * kBlock + nl;
  const bool valid = n < a.N;
  const int HW = a.grid_h * a.grid_w;
  const int pos = part == 0 ? n / HW : (part == 1 ? (n / a.grid_w) % a.grid_h : n % a.grid_w);
  const int off = part == 0 ? 0 : (part == 1 ? D0 : D0 + D1);
  const float* cos_a = part == 0 ? a.cos_t : (part == 1 ? a.cos_h : a.cos_w);
  const float* sin_a = part == 0 ? a.sin_t : (part == 1 ? a.sin_h : a.sin_w);
  const size_t head_tok = (size_t)bh * a.N;
  const bool fallback = a.fallback.test(bh);

  if (fallback) {
#pragma unroll 1
    for (int s = 0; s < 2; ++s) {
      const uint16_t* row = (s == 0 ? a.q : a.k) + (head_tok + (valid ? n : 0)) * D;
      uint16_t* out_row = (s == 0 ? a.q_rope : a.k_rope) + (head_tok + (valid ? n : 0)) * D;
      if (part == 0)
        rope_only_part<D0>(row, valid, cos_a, sin_a, pos, off, out_row);
      else
        rope_only_part<D1>(row, valid, cos_a, sin_a, pos, off, out_row);
    }
    return;
  }

  const size_t pad_row = ((size_t)bh * a.NB + blk) * kBlock;   // first packed row of this block
#pragma unroll 1
  for (int s = 0; s < 2; ++s) {
    const uint16_t* row = (s == 0 ? a.q : a.k) + (head_tok + (valid ? n : 0)) * D;
    float scale;
    if (part == 0)
      qk_part<D0>(row, valid, cos_a, sin_a, pos, off, a.rot64, red, codes, nl, scale);
    else
      qk_part<D1>(row, valid, cos_a, sin_a, pos, off, a.rot64 + part * 4096, red, codes, nl,
                  scale);
    __syncthreads();
    store_qk_codes<D>(codes, (s == 0 ? a.q4 : a.k4) + pad_row * (D / 2));
    if (threadIdx.x == 0) {
      if (s == 0)
        a.q_scale_l2[(size_t)bh * a.NB + blk] = scale * a.kappa;
      else
        a.k_scale[(size_t)bh * a.NB + blk] = scale;
    }
    __syncthreads();
  }

  {
    const uint16_t* row = a.v + (head_tok + (valid ? n : 0)) * D;
    float scale;
    if (part == 0)
      v_part<D0>(row, valid, off, red, codes, nl, scale);
    else
      v_part<D1>(row, valid, off, red, codes, nl, scale);
    __syncthreads();
    store_v_codes<D>(codes, a.v4 + ((size_t)bh * a.NB + blk) * D * 64);
    if (threadIdx.x == 0) a.v_scale[(size_t)bh * a.NB + blk] = scale;
  }
}

hipError_t launch_prologue(int D, int dt, int BH, const PrologueArgs& a, hipStream_t st) {
  dim3 grid(a.NB, BH);
  if (D == 128 && dt == 44)
    hipLaunchKernelGGL((k_prologue<128, 44, 42>), grid, dim3(kThreads), 0, st, a);
  else if (D == 64 && dt == 24)
    hipLaunchKernelGGL((k_prologue<64, 24, 20>), grid, dim3(kThreads), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rotattn

// Internal declarations shared by the HIP translation units of librotattn.so.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rotattn.h"

namespace rotattn {

constexpr int kBlock = ROTATTN_BLOCK;          // tokens per quantization block / key tile
constexpr int kHeadWords = ROTATTN_MAX_HEADS / 32;

// Head-selection bitmask passed by value as a kernel argument.
struct HeadBits {
  uint32_t w[kHeadWords];
  __host__ __device__ bool test(int bh) const { return (w[bh >> 5] >> (bh & 31)) & 1u; }
};

// The value held by lane ^ 32 of this wave (the other 32-lane half):
// ds_bpermute reads lane (byte address / 4) mod 64, so the thread index needs
// no masking.  Cheaper than __shfl_xor, whose generic width handling costs
// extra VALU per call.
__device__ __forceinline__ int other_half(int v) {
  return __builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32u) << 2), v);
}
__device__ __forceinline__ float other_half(float v) {
  return __int_as_float(other_half(__float_as_int(v)));
}

// Max of floats that are never NaN, as single v_max3 / v_max instructions
// (fmaxf must quiet signalling NaNs of operands the compiler cannot prove
// canonical, such as MFMA results, which costs a v_max per chain).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(|a|, |b|, |c|) with the absolute values as input modifiers
__device__ __forceinline__ float vmax3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Nibble layout of a packed INT4 dword: 8 elements e0..e7, byte i holds e_i in
// its low nibble and e_{i+4} in its high nibble.  The two unpack steps below
// give e0..e3 and e4..e7 as int8 lanes holding 16*e (exact: |16*e| <= 112),
// so an i8 MFMA over unpacked operands accumulates 256*I (two unpacked
// operands) or 16*I (one unpacked operand against unscaled int8).
__device__ __forceinline__ uint32_t unpack_lo(uint32_t p) { return (p << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t unpack_hi(uint32_t p) { return p & 0xF0F0F0F0u; }

// Pack 8 int8 codes (two dwords, e0..e3 and e4..e7) into one nibble dword.
__device__ __forceinline__ uint32_t pack_nibbles(uint32_t lo4, uint32_t hi4) {
  return (lo4 & 0x0F0F0F0Fu) | ((hi4 & 0x0F0F0F0Fu) << 4);
}

// Element strides of a [B][H][N][D] fp16 tensor with unit channel stride.
struct Strides {
  int64_t batch, head, token;
  __host__ __device__ int64_t head_offset(int bh, int H) const {
    return (int64_t)(bh / H) * batch + (int64_t)(bh % H) * head;
  }
};

struct PrologueArgs {
  const uint16_t *q, *k, *v;
  Strides in;                   // of q, k and v
  int H;
  const float *cos_t, *sin_t, *cos_h, *sin_h, *cos_w, *sin_w;
  const float *cs_t, *cs_h, *cs_w;   // the same tables as (cos, sin) pairs (library scratch)
  const double* rot64;          // rotation in fp64, [k][r] per partition (t at 0, h at d_t^2, w next);
                                // unused by the kernels without a dense rotation
  uint8_t *q4, *k4, *v4;
  float *q_scale_l2, *k_scale, *v_scale;
  uint16_t *q_rope, *k_rope, *v_t;   // fallback heads: [BH][N_pad][D], V^T tiles
  int N, NB, grid_h, grid_w;
  float kappa;
  HeadBits fallback;            // bit set: RoPE'd fp16 only
};

struct Int4Args {
  const uint8_t *q4, *k4, *v4;
  const float *q_scale_l2, *k_scale, *v_scale;
  uint16_t* o;
  Strides os;                   // of o
  int H;
  int N, NB;
  float log2_15;                // fl32(log2(15))
  float tau[15];                // P-code thresholds
  bool code_sum;                // normalizer: sum of the P codes (FP8/FP6 layouts) instead of sum 2^x
  bool f6;                      // FP6 layout: Q, K, V codes as FP6 E2M3 (else FP8 E4M3)
  HeadBits run;                 // bit set: run this head
};

struct Int4Debug {
  int32_t* s_int;
  uint8_t* p_code;
  int32_t* pv_int;
  float *m_final, *l_final;
  int bh, q_block;
};

struct Fp16Args {
  const uint16_t *q, *k;   // RoPE'd Q', K': [heads][N_pad][D], rows >= N zero
  const uint16_t* v_t;     // V^T per 64-key tile: [heads][N_pad/64][D][64], operand order
  uint16_t* o;
  Strides os;              // of o
  int H;
  int N, NB;
  float kappa;
  HeadBits run;            // by global head index
  int bh0;                 // global index of the heads' first (buffers hold heads bh0..)
};

// Staging of caller fp16 Q', K', V for the FP16 attention (heads bh0.. of a chunk).
struct StageArgs {
  const uint16_t *q, *k, *v;
  Strides in;              // of q, k and v
  int H, N, NB;
  uint16_t *q_pad, *k_pad, *v_t;   // [chunk heads][N_pad][D] each (v_t as V^T tiles)
  HeadBits run;            // by global head index
  int bh0;
};

// The library scratch of a rotattn_prepared (rot64): the rotation in fp64
// [k][r] per partition from byte 0; from byte kRotFragOffset the prologue's
// MFMA B fragments of it in fp32, 64 lanes x kRotFragStride floats per
// partition; from byte kRotTabOffset the RoPE tables as (cos, sin) pairs, axis
// t, then h, then w, each [position][channel pair].
constexpr int kRotFragOffset = 48 * 1024;
constexpr int kRotFragStride = 36;
constexpr int kRotTabOffset = 96 * 1024;
static_assert(kRotFragOffset >= (44 * 44 + 2 * 42 * 42) * 8, "fp64 rotation before the fragments");
static_assert(kRotFragOffset + 3 * 64 * kRotFragStride * 4 <= kRotTabOffset, "fragments fit");

// The QKV projection with the prologue as its epilogue: x [B][N][C] (channel
// stride 1) times the fused weight w [3 H D][C] (row r = output channel r: Q
// heads, then K, then V), + bias, rounded to fp16, then the prologue's work on
// each 128-token x 128-channel tile.  Work-group tiles are grouped 8 token
// blocks x 8 (tensor, head) pairs per XCD.
struct QkvProjArgs {
  const uint16_t* x;
  int64_t x_batch, x_token;     // element strides of x
  const uint16_t* w;
  const uint16_t* bias;         // [3 H D] or null
  uint16_t* qkv_out;            // optional [3][B H][N_pad][D] copy of the projection, or null
  int C, B;
  int SBT, SHT;                 // tile groups along tokens and along (tensor, head) pairs
  int last_block_only;          // 128 x 128 kernel: only the last block of each batch entry
  PrologueArgs p;               // q, k, v and in unused
};

// Launchers (each defined next to its kernel).  Return a hipError_t.
hipError_t launch_rot_to_f64(const float* rt, const float* rh, const float* rw, int dt, int dh,
                             double* out, hipStream_t st);
hipError_t launch_rope_pairs(const rotattn_rope_rot* rr, int np_t, int np_h, int np_w, float* out,
                             hipStream_t st);
hipError_t launch_prologue(int D, int dt, int BH, int layout, bool rot, const PrologueArgs& a,
                           hipStream_t st);
hipError_t launch_int4(int D, int BH, const Int4Args& a, const Int4Debug* dbg, hipStream_t st);
hipError_t launch_int4_f8(int D, int BH, const Int4Args& a, const Int4Debug* dbg, hipStream_t st);
hipError_t launch_fp16(int D, int BH, const Fp16Args& a, hipStream_t st);
hipError_t launch_stage_fp16(int D, int nbh, const StageArgs& a, hipStream_t st);
hipError_t launch_qkv_proj(int D, int dt, int layout, bool rot, const QkvProjArgs& a,
                           hipStream_t st);
hipError_t launch_pcode_sweep(bool f8, uint32_t mag_lo, uint32_t count, const float tau[15],
                              float log2_15, uint32_t* transitions, uint32_t max_transitions,
                              uint32_t* n_trans, hipStream_t st);
hipError_t launch_pcode_eval(bool f8, const int32_t* I, uint32_t n, float c, float m,
                             const float tau[15], float log2_15, uint8_t* codes, hipStream_t st);

}  // namespace rotattn

// K3: FP16 FlashAttention forward on gfx950 -- RotateAttention's selective
// FP16 fallback (RotateAttention page, Abstract: accuracy-sensitive attention
// runs in FP16 instead of INT4).  Inputs are the RoPE'd fp16 Q', K' (no
// rotation, no quantization) and fp16 V; O = softmax(Q'K'^T/sqrt(D)) V.
//
// One work-group = 4 waves x 32 queries; 64-key tiles staged through LDS
// (double buffered, one barrier per tile).  S^T = K Q'^T on
// v_mfma_f32_32x32x16_f16, fp32 online softmax in the log2 domain (kappa =
// log2(e)/sqrt(D)), P rounded to fp16 in registers and used directly as the
// P^T operand of O^T = V^T P^T (same orientation trick as the INT4 kernel).
// V is transposed into LDS while staging, with the key order of each 32-key
// subtile permuted to match the P^T operand layout.
#include <math.h>

#include "rotattn_internal.h"

namespace rotattn {

constexpr int kFThreads = 256;
constexpr int kKT = 64;                   // keys per tile
constexpr int kFVStride = 2 * kKT + 16;   // V^T row in LDS: 64 keys fp16 + 16 bytes

template <int D>
struct Fp16Kernel {
  static constexpr int KS = D / 16;         // k-steps of 16 channels
  static constexpr int DB = D / 32;
  static constexpr int KStride = 2 * D + 16;
  static constexpr int KPT = D / 2;         // K tile bytes per thread (64 keys x 2D bytes / 256)
  static constexpr int VITEMS = 16 * (D / 8);   // (4-key chunk, 8-channel chunk) items per tile

  template <bool TAIL>
  __device__ __forceinline__ static void tile(const Fp16Args& a, int t, const uint8_t* sk,
                                              const uint8_t* sv, const v8h (&qf)[KS], float& m,
                                              float& l, v16f (&O)[DB]) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, hh = lane >> 5;
    v16f S[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      S[sub] = v16f{0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v8h kf = *(const v8h*)(sk + (32 * sub + col) * KStride + 2 * (16 * ks + 8 * hh));
        S[sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], S[sub], 0, 0, 0);
      }
    }
    if (TAIL) {
      const int nv = a.N - t * kKT;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3) >= nv) S[sub][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[sub][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx * a.kappa);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    v8h P[2][2];
    float ls = 0.0f;   // tile sum first, then into the running l (see the INT4 kernel)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[sub][r], a.kappa, -mnew));
        ls += p;
        P[sub][r >> 3][r & 7] = (_Float16)p;
      }
    l = fmaf(l, alpha, ls);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const v8h vf =
              *(const v8h*)(sv + (32 * db + col) * kFVStride + 2 * (32 * sub + 16 * s + 8 * hh));
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, P[sub][s], O[db], 0, 0, 0);
        }
  }

  __device__ static void run(const Fp16Args& a) {
    __shared__ __align__(16) uint8_t sk[2][kKT * KStride];
    __shared__ __align__(16) uint8_t sv[2][D * kFVStride];
    const int qb = blockIdx.x, bh = blockIdx.y;
    if (!a.run.test(bh)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int N = a.N;
    const size_t head = (size_t)bh * N;   // first token row of this head

    v8h qf[KS];
    {
      const int query = qb * kBlock + 32 * w + col;
      const uint16_t* qrow = a.q + (head + (query < N ? query : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 p = query < N ? *(const uint4*)(qrow + 16 * ks + 8 * hh) : uint4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(v8h, p);
      }
    }

    uint4 kreg[KPT / 16];
    uint4 vreg[4 * ((VITEMS + kFThreads - 1) / kFThreads)];
    auto gload = [&](int t) {
      {
        const int key = t * kKT + (tid >> 2);
        const uint8_t* src = (const uint8_t*)(a.k + (head + (key < N ? key : 0)) * D) + (tid & 3) * KPT;
#pragma unroll
        for (int i = 0; i < KPT / 16; ++i)
          kreg[i] = key < N ? *(const uint4*)(src + 16 * i) : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int it = 0; it < (VITEMS + kFThreads - 1) / kFThreads; ++it) {
        const int item = tid + it * kFThreads;
        if (item < VITEMS) {
          const int dc = item % (D / 8), qc = item / (D / 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t * kKT + 4 * qc + i;
            vreg[4 * it + i] = key < N ? *(const uint4*)(a.v + (head + key) * D + 8 * dc)
                                       : uint4{0, 0, 0, 0};
          }
        }
      }
    };
    auto lstore = [&](int buf) {
      {
        uint8_t* dst = sk[buf] + (tid >> 2) * KStride + (tid & 3) * KPT;
#pragma unroll
        for (int i = 0; i < KPT / 16; ++i) *(uint4*)(dst + 16 * i) = kreg[i];
      }
#pragma unroll
      for (int it = 0; it < (VITEMS + kFThreads - 1) / kFThreads; ++it) {
        const int item = tid + it * kFThreads;
        if (item < VITEMS) {
          const int dc = item % (D / 8), qc = item / (D / 8);
          // 4-key chunk c of a 32-key subtile goes to chunk position with its
          // two low bits swapped: the P^T operand of k-step s, lane half hh
          // holds keys 16s + 8(j/4) + 4hh + j%4, j = 0..7.
          const int c = qc & 7;
          const int pos = (qc & ~7) | (c & 4) | ((c & 1) << 1) | ((c >> 1) & 1);
          const uint32_t* r0 = (const uint32_t*)&vreg[4 * it];
          const uint32_t* r1 = (const uint32_t*)&vreg[4 * it + 1];
          const uint32_t* r2 = (const uint32_t*)&vreg[4 * it + 2];
          const uint32_t* r3 = (const uint32_t*)&vreg[4 * it + 3];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint2 even{__builtin_amdgcn_perm(r1[e], r0[e], 0x05040100u),
                             __builtin_amdgcn_perm(r3[e], r2[e], 0x05040100u)};
            const uint2 odd{__builtin_amdgcn_perm(r1[e], r0[e], 0x07060302u),
                            __builtin_amdgcn_perm(r3[e], r2[e], 0x07060302u)};
            *(uint2*)(sv[buf] + (8 * dc + 2 * e) * kFVStride + 8 * pos) = even;
            *(uint2*)(sv[buf] + (8 * dc + 2 * e + 1) * kFVStride + 8 * pos) = odd;
          }
        }
      }
    };

    float m = -INFINITY, l = 0.0f;
    v16f O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = v16f{0.0f};
    const int NT = (N + kKT - 1) / kKT;
    gload(0);
    lstore(0);
    __syncthreads();
    // full tiles in the loop, the last (possibly ragged) tile peeled off
#pragma unroll 1
    for (int t = 0; t < NT - 1; ++t) {
      const int buf = t & 1;
      gload(t + 1);
      tile<false>(a, t, sk[buf], sv[buf], qf, m, l, O);
      lstore(buf ^ 1);
      __syncthreads();
    }
    {
      const int t = NT - 1, buf = t & 1;
      if ((N % kKT) != 0)
        tile<true>(a, t, sk[buf], sv[buf], qf, m, l, O);
      else
        tile<false>(a, t, sk[buf], sv[buf], qf, m, l, O);
    }
    l += __shfl_xor(l, 32, 64);
    const int query = qb * kBlock + 32 * w + col;
    if (query < N) {
      const float il = 1.0f / l;
      uint16_t* orow = a.o + (head + query) * D;
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

template <int D>
__global__ __launch_bounds__(kFThreads, 2) void k_fp16_attn(Fp16Args a) {
  Fp16Kernel<D>::run(a);
}

hipError_t launch_fp16(int D, int BH, const Fp16Args& a, hipStream_t st) {
  dim3 grid((a.N + kBlock - 1) / kBlock, BH);
  if (D == 128)
    hipLaunchKernelGGL(k_fp16_attn<128>, grid, dim3(kFThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_fp16_attn<64>, grid, dim3(kFThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace rotattn

// K3: FP16 FlashAttention forward on gfx950 -- RotateAttention's selective
// FP16 fallback (RotateAttention page, Abstract: accuracy-sensitive attention
// runs in FP16 instead of INT4).  Inputs are the prologue's fallback buffers:
// RoPE'd fp16 Q', K' (no rotation, no quantization; rows padded to N_pad with
// zeros) and V^T per 64-key tile in the operand order of the P.V product.
// O = softmax(Q'K'^T/sqrt(D)) V.
//
// One work-group = 8 waves x 32 queries, one per CU (two waves per SIMD, so
// that one wave's softmax overlaps the other's MFMAs); the 8 waves share every
// K and V^T tile the work-group brings into LDS (4-wave work-groups, two per
// CU, moved twice the tile bytes per flop and ran 1.5% slower).  Per 64-key
// tile: S^T = K Q'^T on v_mfma_f32_32x32x16_f16 (each lane then holds one
// query's scores in the layout of the P^T operand), fp32 online softmax in the
// log2 domain (kappa = log2(e)/sqrt(D)), P rounded to fp16 in registers,
// O^T += V^T P^T.  K and V^T tiles go straight from HBM into XOR-swizzled LDS
// (global_load_lds, 64-bank layout), double buffered; the next tile is
// requested after the softmax, while P.V runs; MFMA blocks run at raised wave
// priority.
#include <math.h>

#include "rotattn_internal.h"

namespace rotattn {

constexpr int kFThreads = 512;   // 8 waves: 256 queries per work-group
constexpr int kKT = 64;   // keys per tile

typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

template <int D>
struct Fp16Kernel {
  static constexpr int KS = D / 16;              // k-steps of 16 channels for QK^T
  static constexpr int DB = D / 32;              // 32-channel blocks of O^T
  static constexpr int NW = kFThreads / 64;
  static constexpr int KRB = 2 * D;              // bytes per K row
  static constexpr int KCPR = KRB / 16;          // 16-byte chunks per K row
  static constexpr int KRPB = 256 / KRB;         // K rows per 256 bytes (one bank row)
  static constexpr int TCH = kKT * KRB / 16;     // chunks per tile (K and V^T alike)
  static constexpr int LOADS = TCH / kFThreads;  // loads per thread per tile and tensor
  static_assert(TCH % kFThreads == 0 && D * 128 / 16 == TCH, "whole waves per tile");

  // XOR swizzle of the 16-byte chunks of a row: the 16 rows read together by
  // a ds_read_b128 land on 16 different chunk columns of the 64 banks
  __device__ __forceinline__ static int kswz(int row) { return (row / KRPB) & (KCPR - 1); }
  __device__ __forceinline__ static int vswz(int row) { return (row >> 1) & 7; }   // 128-byte rows

  __device__ __forceinline__ static v8h ld16(const uint8_t* p) { return *(const v8h*)p; }

  __device__ __forceinline__ static void qk(const uint8_t* sk, const v8h (&qf)[KS], v16f (&S)[2]) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = 32 * sub + col;
      S[sub] = v16f{0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        S[sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            ld16(sk + row * KRB + 16 * ((2 * ks + hh) ^ kswz(row))), qf[ks], S[sub], 0, 0, 0);
    }
  }

  __device__ __forceinline__ static void pv(const uint8_t* sv, const v8h (&P)[2][2],
                                            v16f (&O)[DB]) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 32 * db + col;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              ld16(sv + row * 128 + 16 * ((4 * sub + 2 * s + hh) ^ vswz(row))), P[sub][s], O[db],
              0, 0, 0);
    }
  }

  // Keys >= nv (last tile only) get S = -inf.
  __device__ __forceinline__ static void mask_tail(v16f (&S)[2], int nv) {
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * sub + 8 * (r >> 2) + 4 * hh + (r & 3) >= nv) S[sub][r] = -INFINITY;
  }

  __device__ __forceinline__ static void softmax(const Fp16Args& a, v16f (&S)[2], float& m,
                                                 float& l, v16f (&O)[DB], v8h (&P)[2][2]) {
    // scores of finite fp16 inputs are never NaN: plain v_max3 chains
    float mx = vmax3(S[0][0], S[0][1], S[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = vmax3(mx, S[0][r], S[0][r + 1]);
    mx = vmax3(mx, S[0][15], S[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) mx = vmax3(mx, S[1][r], S[1][r + 1]);
    mx = vmax2(mx, S[1][15]);
    mx = vmax2(mx, other_half(mx));
    const float mnew = vmax2(m, mx * a.kappa);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    // the running max moves in a minority of tiles (mostly the first ones)
    if (__builtin_expect(__ballot(alpha != 1.0f) != 0, 0)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    float ls = 0.0f;   // tile sum first, then into the running l
    // The fused S kappa - m' compares an exact product with the rounded one in
    // m' = fl(max S kappa): past |m'| = 2^12 that difference could reach whole
    // units and overflow the exponential, so such a wave (logits of thousands
    // of nats) takes fl(fl(S kappa) - m') <= 0 instead.
    const bool exact_arg = __ballot(fabsf(mnew) > 4096.0f) != 0;
    float e[2][16];
    if (__builtin_expect(!exact_arg, 1)) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) e[sub][r] = __builtin_amdgcn_exp2f(fmaf(S[sub][r], a.kappa, -mnew));
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) e[sub][r] = __builtin_amdgcn_exp2f(S[sub][r] * a.kappa - mnew);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t wpk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * s + 2 * i;
          const float p0 = e[sub][r];
          const float p1 = e[sub][r + 1];
          ls += p0;
          ls += p1;
          // one v_cvt_pk_f16_f32 per pair (round to nearest even), packed in place
          wpk[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){p0, p1}, v2h));
        }
        P[sub][s] = __builtin_bit_cast(v8h, uint4{wpk[0], wpk[1], wpk[2], wpk[3]});
      }
    l = fmaf(l, alpha, ls);
  }

  __device__ static void run(const Fp16Args& a) {
    // two K and two V^T buffers as separate arrays, selected at compile time:
    // the compiler then sees that a tile load and the LDS reads of the other
    // buffer do not overlap and does not wait for the load before them
    __shared__ __align__(16) uint8_t sk0[kKT * KRB], sk1[kKT * KRB];
    __shared__ __align__(16) uint8_t sv0[D * 128], sv1[D * 128];
    // bh: the head in the buffers; the run mask and O use its global index
    const int qb = blockIdx.x, bh = blockIdx.y, gbh = a.bh0 + bh;
    if (!a.run.test(gbh)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int N = a.N, NT = (N + kKT - 1) / kKT;
    const size_t head_pad = (size_t)bh * a.NB * kBlock;   // first padded row of this head

    v8h qf[KS];
    {
      // queries past N (the last work-group's second half when N_pad / 128 is
      // odd) read the last valid row and are not written
      const int qrow_i = qb * (NW * 32) + 32 * w + col;
      const uint16_t* qrow = a.q + (head_pad + (size_t)(qrow_i < N ? qrow_i : N - 1)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const v8h*)(qrow + 16 * ks + 8 * hh);
    }

    // tile loads straight into LDS: wave w, instruction i fills chunks
    // (NW i + w) * 64 + lane of the tile.  Instruction i lands 32 K rows (64
    // V^T rows) further down than instruction 0 and the swizzle keys repeat
    // with periods dividing that, so its per-lane byte offset is instruction
    // 0's plus 8 KiB i: the uniform part goes to the scalar base (saddr form) and one
    // 32-bit offset register per tensor remains.
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    constexpr uint32_t kInstr = NW * 64 * 16;   // bytes per load instruction of the work-group
    uint32_t koff0, voff0;
    {
      const int pc = w * 64 + lane;   // physical chunk of instruction 0
      const int krow = pc / KCPR, vrow = pc / 8;
      koff0 = krow * KRB + 16 * ((pc % KCPR) ^ kswz(krow));
      voff0 = vrow * 128 + 16 * ((pc % 8) ^ vswz(vrow));
    }
    auto gloadK = [&](int t, uint8_t* dst) {
      const uint8_t* kb = (const uint8_t*)(a.k + (head_pad + (size_t)t * kKT) * D);
      // opaque per tile: keeps the loop from turning base + offset into
      // per-lane 64-bit pointers held in registers
      uint32_t ko = koff0;
      asm volatile("" : "+v"(ko));
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint8_t* kbi = kb + kInstr * i;
        asm volatile("" : "+s"(kbi));
        __builtin_amdgcn_global_load_lds((const void*)(kbi + ko),
                                         (lds_ptr)(dst + (NW * i + wu) * 1024), 16, 0, 0);
      }
    };
    auto gloadV = [&](int t, uint8_t* dst) {
      const uint8_t* vb = (const uint8_t*)(a.v_t + (head_pad + (size_t)t * kKT) * D);
      uint32_t vo = voff0;
      asm volatile("" : "+v"(vo));
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint8_t* vbi = vb + kInstr * i;
        asm volatile("" : "+s"(vbi));
        __builtin_amdgcn_global_load_lds((const void*)(vbi + vo),
                                         (lds_ptr)(dst + (NW * i + wu) * 1024), 16, 0, 0);
      }
    };

    float m = -INFINITY, l = 0.0f;
    v16f O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = v16f{0.0f};
    const int nv_last = N - (NT - 1) * kKT;

    gloadK(0, sk0);
    gloadV(0, sv0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // tile t in (skc, svc); tile t+1 goes to (skn, svn), last read in tile t-1
    auto step = [&](int t, const uint8_t* skc, const uint8_t* svc, uint8_t* skn, uint8_t* svn) {
      v16f S[2];
      v8h P[2][2];
      __builtin_amdgcn_s_setprio(1);
      qk(skc, qf, S);
      __builtin_amdgcn_s_setprio(0);
      if (__builtin_expect(t == NT - 1 && nv_last < kKT, 0)) {
        // opaque: nv_last is loop-invariant, and the comparisons would be
        // hoisted out of the loop and kept live as SGPR masks
        int nv = nv_last;
        asm volatile("" : "+v"(nv));
        mask_tail(S, nv);
      }
      softmax(a, S, m, l, O, P);
      if (t + 1 < NT) {
        gloadK(t + 1, skn);
        gloadV(t + 1, svn);
      }
      __builtin_amdgcn_s_setprio(1);
      pv(svc, P, O);
      __builtin_amdgcn_s_setprio(0);
      // this thread's tile loads have landed in LDS before anyone passes the barrier
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
#pragma unroll 1
    for (int t = 0; t < NT; t += 2) {
      step(t, sk0, sv0, sk1, sv1);
      if (t + 1 < NT) step(t + 1, sk1, sv1, sk0, sv0);
    }

    l += other_half(l);
    const int query = qb * (NW * 32) + 32 * w + col;
    if (query < N) {
      const float il = 1.0f / l;
      uint16_t* orow = a.o + a.os.head_offset(gbh, a.H) + (int64_t)query * a.os.token;
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
__global__ __launch_bounds__(kFThreads, 1) void k_fp16_attn(Fp16Args a) {
  Fp16Kernel<D>::run(a);
}

// BH: heads in the buffers (global heads a.bh0 .. a.bh0 + BH - 1)
hipError_t launch_fp16(int D, int BH, const Fp16Args& a, hipStream_t st) {
  dim3 grid((a.NB * kBlock + kFThreads / 2 - 1) / (kFThreads / 2), BH);   // 256 queries each
  if (D == 128)
    hipLaunchKernelGGL(k_fp16_attn<128>, grid, dim3(kFThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_fp16_attn<64>, grid, dim3(kFThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace rotattn

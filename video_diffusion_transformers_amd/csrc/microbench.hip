// K4: gfx950 roofline denominators measured on the box -- HBM copy bandwidth,
// i8 and f16 MFMA rates, VALU issue rates of the instructions the softmax and
// P-code path use, and MFMA/VALU co-issue.  Also the plain copy kernel of known
// size against which rocprofv3's FETCH_SIZE / WRITE_SIZE counters are scaled.
//
//   rotattn_microbench [--copy-only] [--copy-mib N]
//
// Prints one JSON object.  Each rate kernel runs a few milliseconds with
// enough independent chains per lane and waves per SIMD to be throughput-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CK(x)                                                                        \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                       \
    }                                                                                \
  } while (0)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                               size_t n) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (; i < n; i += stride) dst[i] = src[i];
}

constexpr int kChains = 8;

#define RATE_KERNEL(NAME, BODY)                                          \
  __global__ __launch_bounds__(256) void NAME(float* out, int iters) {   \
    float a[kChains];                                                    \
    for (int j = 0; j < kChains; ++j) a[j] = 1e-3f * (threadIdx.x + j);  \
    for (int i = 0; i < iters; ++i) {                                    \
      _Pragma("unroll") for (int j = 0; j < kChains; ++j) { BODY; }      \
    }                                                                    \
    float s = 0;                                                         \
    for (int j = 0; j < kChains; ++j) s += a[j];                         \
    if (s == 12345.678f) out[threadIdx.x] = s;                           \
  }

// one instruction per chain step
RATE_KERNEL(k_fma, a[j] = __builtin_fmaf(a[j], 0.999f, -1e-4f))
RATE_KERNEL(k_exp, a[j] = __builtin_amdgcn_exp2f(a[j]))
RATE_KERNEL(k_fract, a[j] = __builtin_amdgcn_fractf(a[j] + 0.37f))
RATE_KERNEL(k_cvt, a[j] = (float)(int)a[j] + 0.5f)

__global__ __launch_bounds__(256) void k_fma64(float* out, int iters) {
  double a[kChains];
  for (int j = 0; j < kChains; ++j) a[j] = 1e-3 * (threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) a[j] = __builtin_fma(a[j], 0.999, -1e-4);
  }
  double s = 0;
  for (int j = 0; j < kChains; ++j) s += a[j];
  if (s == 12345.678) out[threadIdx.x] = (float)s;
}

// LDS read bandwidth: every lane reads 16 bytes per instruction from a 16 KB
// tile (distinct rows per lane, 144-byte row stride as in the attention kernels)
__global__ __launch_bounds__(256) void k_lds(float* out, int iters) {
  __shared__ __align__(16) uint4 tile[1024];
  for (int i = threadIdx.x; i < 1024; i += 256) tile[i] = uint4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  uint4 acc = uint4{0, 0, 0, 0};
  for (int i = 0; i < iters; ++i) {
    // the tile is unchanged across iterations: without this compiler barrier
    // the reads would be loaded once and reused, and no LDS traffic measured
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = ((lane & 31) * 9 + (lane >> 5) + 2 * j + (i & 7)) & 1023;
      const uint4 v = tile[idx];
      acc.x ^= v.x; acc.y += v.y; acc.z ^= v.z; acc.w += v.w;
    }
  }
  if (acc.x == 0x12345u) out[threadIdx.x] = (float)(acc.y + acc.z + acc.w);
}

__global__ __launch_bounds__(256) void k_cvtpk(float* out, int iters) {
  float a[kChains];
  uint32_t acc = 0;
  for (int j = 0; j < kChains; ++j) a[j] = 1e-3f * (threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc = __builtin_amdgcn_cvt_pk_u8_f32(a[j], j & 3, acc);
  }
  if (acc == 0x12345678u) out[threadIdx.x] = (float)acc;
}

__global__ __launch_bounds__(256) void k_mfma_i8(float* out, int iters) {
  v4i a = {(int)threadIdx.x, 1, 2, 3}, b = {3, 2, 1, (int)threadIdx.x};
  v16i c[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
  }
  int s = 0;
  for (int j = 0; j < 4; ++j) for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == 12345) out[threadIdx.x] = (float)s;
}

__global__ __launch_bounds__(256) void k_mfma_f16(float* out, int iters) {
  v8h a, b;
  for (int j = 0; j < 8; ++j) { a[j] = (_Float16)(1e-3f * threadIdx.x); b[j] = (_Float16)0.5f; }
  v16f c[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < 4; ++j) for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == 12345.f) out[threadIdx.x] = s;
}

// co-issue: even waves run the i8 MFMA loop, odd waves an FMA loop
__global__ __launch_bounds__(256) void k_mix(float* out, int iters, int valu_per_mfma) {
  const int wave = threadIdx.x >> 6;
  if (wave & 1) {
    float a[kChains];
    for (int j = 0; j < kChains; ++j) a[j] = 1e-3f * (threadIdx.x + j);
    const int n = iters * valu_per_mfma * 4 / kChains;
    for (int i = 0; i < n; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) a[j] = __builtin_fmaf(a[j], 0.999f, -1e-4f);
    }
    float s = 0;
    for (int j = 0; j < kChains; ++j) s += a[j];
    if (s == 12345.678f) out[threadIdx.x] = s;
  } else {
    v4i a = {(int)threadIdx.x, 1, 2, 3}, b = {3, 2, 1, (int)threadIdx.x};
    v16i c[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
    }
    int s = 0;
    for (int j = 0; j < 4; ++j) for (int r = 0; r < 16; ++r) s += c[j][r];
    if (s == 12345) out[threadIdx.x] = (float)s;
  }
}

static float time_ms(void (*launch)(void*), void* ctx, int reps) {
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  launch(ctx);
  CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0));
  for (int r = 0; r < reps; ++r) launch(ctx);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ms;
  CK(hipEventElapsedTime(&ms, e0, e1));
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return ms / reps;
}

struct RateCtx {
  void (*kern)(float*, int);
  float* out;
  int iters, blocks;
};
static void launch_rate(void* p) {
  RateCtx* c = (RateCtx*)p;
  hipLaunchKernelGGL(c->kern, dim3(c->blocks), dim3(256), 0, 0, c->out, c->iters);
}
// MFMA and VALU work in the same wave: each step is one i8 32x32x32 MFMA
// (four independent accumulators) and N independent v_fma_f32 (eight
// chains).  Clocks per step against the MFMA alone and N FMAs alone show how
// much of the matrix core's time can hide vector work on one SIMD.
template <int N>
__global__ __launch_bounds__(256) void k_mix_same(float* out, int iters) {
  v4i a = {(int)threadIdx.x, 1, 2, 3}, b = {3, 2, 1, (int)threadIdx.x};
  v16i c[4] = {};
  float f[kChains];
  for (int j = 0; j < kChains; ++j) f[j] = 1e-3f * (threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < N; ++r) f[r % kChains] = __builtin_fmaf(f[r % kChains], 0.999f, -1e-4f);
    }
  }
  int s = 0;
  for (int j = 0; j < 4; ++j) for (int r = 0; r < 16; ++r) s += c[j][r];
  float t = 0;
  for (int j = 0; j < kChains; ++j) t += f[j];
  if (s == 12345 || t == 1.2345f) out[threadIdx.x] = t + (float)s;
}

// v_exp_f32 and independent vector work in the same wave: per step one
// exponential (eight chains) and N v_fma_f32 on eight other chains.  Clocks per
// step against the exponential alone and N FMAs alone show whether the
// exponential's issue cost overlaps other VALU work.
template <int N>
__global__ __launch_bounds__(256) void k_exp_mix(float* out, int iters) {
  float e[kChains], f[kChains];
  for (int j = 0; j < kChains; ++j) {
    e[j] = -1e-3f * (threadIdx.x + j);
    f[j] = 1e-3f * (threadIdx.x + j);
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      e[j] = __builtin_amdgcn_exp2f(e[j]);
#pragma unroll
      for (int r = 0; r < N; ++r) {
        const int c = (j * N + r) % kChains;
        f[c] = __builtin_fmaf(f[c], 0.999f, -1e-4f);
      }
    }
  }
  float s = 0;
  for (int j = 0; j < kChains; ++j) s += e[j] + f[j];
  if (s == 12345.678f) out[threadIdx.x] = s;
}

// v_exp_f32 in one wave and v_fma_f32 in another: even waves of a
// work-group run exponentials (eight chains), odd waves FMAs; time against
// each kind alone shows whether the exponentials of one wave overlap the
// vector work of another on the same SIMD.
__global__ __launch_bounds__(256) void k_exp_fma_waves(float* out, int iters, int mode) {
  const int wave = threadIdx.x >> 6;
  // mode 0: both kinds; 1: exponential waves only; 2: FMA waves only
  const bool run_exp = (wave & 1) == 0 && mode != 2;
  const bool run_fma = (wave & 1) == 1 && mode != 1;
  float a[kChains];
  for (int j = 0; j < kChains; ++j) a[j] = -1e-3f * (threadIdx.x + j);
  if (run_exp) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) a[j] = __builtin_amdgcn_exp2f(a[j]);
    }
  } else if (run_fma) {
    for (int i = 0; i < iters * 3; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) a[j] = __builtin_fmaf(a[j], 0.999f, -1e-4f);
    }
  }
  float s = 0;
  for (int j = 0; j < kChains; ++j) s += a[j];
  if (s == 12345.678f) out[threadIdx.x] = s;
}

// FP8 MFMA waves beside vector waves of one instruction kind (OP 0: v_fma_f32,
// 1: v_exp_f32, 2: v_max3_f32, 3: v_mul_f32): even waves of a work-group run
// 32x32x64 FP8 MFMAs (four accumulators), odd waves VPM vector instructions
// per MFMA.  mode 0: both, 1: MFMA waves only, 2: vector waves only.
template <int OP>
__global__ __launch_bounds__(256) void k_mix_f8(float* out, int iters, int vpm, int mode) {
  const int wave = threadIdx.x >> 6;
  if ((wave & 1) == 0) {
    if (mode == 2) return;
    v8i a = {(int)threadIdx.x, 1, 2, 3, 4, 5, 6, 7}, b = {7, 6, 5, 4, 3, 2, 1, (int)threadIdx.x};
    v16f c[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
    }
    float s = 0;
    for (int j = 0; j < 4; ++j) for (int r = 0; r < 16; ++r) s += c[j][r];
    if (s == 12345.f) out[threadIdx.x] = s;
  } else {
    if (mode == 1) return;
    float a[kChains];
    for (int j = 0; j < kChains; ++j) a[j] = -1e-3f * (threadIdx.x + j);
    const int n = iters * vpm * 4 / kChains;
    for (int i = 0; i < n; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) {
        if (OP == 0) a[j] = __builtin_fmaf(a[j], 0.999f, -1e-4f);
        if (OP == 1) a[j] = __builtin_amdgcn_exp2f(a[j]);
        if (OP == 2) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(a[j]) : "v"(a[(j + 1) % kChains]), "v"(a[(j + 2) % kChains]));
        if (OP == 3) a[j] = a[j] * 0.999f;
      }
    }
    float s = 0;
    for (int j = 0; j < kChains; ++j) s += a[j];
    if (s == 12345.678f) out[threadIdx.x] = s;
  }
}

// v_rndne_f32 (opaque, so that rint(rint(x)) is not folded)
RATE_KERNEL(k_rndne, asm volatile("v_rndne_f32 %0, %0" : "+v"(a[j])))

// v_cvt_pk_fp8_f32: two floats -> two FP8 bytes (eight independent outputs)
__global__ __launch_bounds__(256) void k_cvt_fp8(float* out, int iters) {
  float a[kChains];
  uint32_t acc[kChains];
  for (int j = 0; j < kChains; ++j) {
    a[j] = 1e-3f * (threadIdx.x + j);
    acc[j] = 0;
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_cvt_pk_fp8_f32(a[j], a[(j + 1) % kChains], acc[j], false);
  }
  uint32_t s = 0;
  for (int j = 0; j < kChains; ++j) s ^= acc[j];
  if (s == 0x12345678u) out[threadIdx.x] = (float)s;
}

// v_cvt_scalef32_2xpk16_fp6_f32: 32 floats -> 32 FP6 (E2M3) values in six
// dwords per instruction; four independent outputs per step
typedef int v6i __attribute__((ext_vector_type(6)));
__global__ __launch_bounds__(256) void k_cvt_fp6(float* out, int iters) {
  v16f x, y;
  for (int j = 0; j < 16; ++j) {
    x[j] = 0.5f * ((threadIdx.x + j) & 15);
    y[j] = 0.25f * ((threadIdx.x + 3 * j) & 15);
  }
  uint32_t s = 0;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // opaque inputs: every conversion is issued (none is merged with another)
      asm volatile("" : "+v"(x), "+v"(y));
      const v6i r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(x, y, 1.0f);
      s ^= (uint32_t)r[j];
    }
  }
  if (s == 0x12345678u) out[threadIdx.x] = (float)s;
}

// 32x32x64 f8f6f4 MFMA with operand formats FA (A) and FB (B): 0 = FP8 E4M3,
// 2 = FP6 E2M3 (six of the eight operand dwords are read)
template <int FA, int FB>
__global__ __launch_bounds__(256) void k_mfma_f8f6f4(float* out, int iters) {
  v8i a = {(int)threadIdx.x, 1, 2, 3, 4, 5, 6, 7}, b = {7, 6, 5, 4, 3, 2, 1, (int)threadIdx.x};
  v16f c[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], FA, FB, 0, 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < 4; ++j) for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == 12345.f) out[threadIdx.x] = s;
}

struct MixCtx {
  float* out;
  int iters, blocks, vpm;
};
static void launch_mix(void* p) {
  MixCtx* c = (MixCtx*)p;
  hipLaunchKernelGGL(k_mix, dim3(c->blocks), dim3(256), 0, 0, c->out, c->iters, c->vpm);
}
struct CopyCtx {
  const uint4* src;
  uint4* dst;
  size_t n;
};
static void launch_copy(void* p) {
  CopyCtx* c = (CopyCtx*)p;
  hipLaunchKernelGGL(k_copy, dim3(256 * 32), dim3(256), 0, 0, c->src, c->dst, c->n);
}

int main(int argc, char** argv) {
  bool copy_only = false;
  size_t copy_mib = 4096;
  for (int i = 1; i < argc; ++i) {
    if (!strcmp(argv[i], "--copy-only")) copy_only = true;
    else if (!strcmp(argv[i], "--copy-mib") && i + 1 < argc) copy_mib = (size_t)atol(argv[++i]);
  }
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  printf("{\"device\": \"%s\", \"cus\": %d", prop.gcnArchName, cus);

  const size_t bytes = copy_mib << 20;
  uint4 *src, *dst;
  CK(hipMalloc(&src, bytes));
  CK(hipMalloc(&dst, bytes));
  CK(hipMemset(src, 1, bytes));
  CopyCtx cc{src, dst, bytes / 16};
  const float cms = time_ms(launch_copy, &cc, copy_only ? 3 : 10);
  printf(", \"copy_bytes_each_way\": %zu, \"copy_ms\": %.4f, \"copy_GBps\": %.1f", bytes, cms,
         2.0 * bytes / (cms * 1e-3) / 1e9);
  CK(hipFree(src));
  CK(hipFree(dst));
  if (copy_only) {
    printf("}\n");
    return 0;
  }

  float* out;
  CK(hipMalloc(&out, 1024 * sizeof(float)));
  const int blocks = cus * 8;   // 8 waves per SIMD
  struct {
    const char* name;
    void (*k)(float*, int);
    double per_iter;   // lane-ops per lane per iteration
  } vk[] = {{"fma", k_fma, kChains}, {"exp", k_exp, kChains},
            {"add_fract_steps", k_fract, kChains},        // v_add + v_fract per step
            {"cvt_cvt_add_steps", k_cvt, kChains},        // f32->i32, i32->f32, v_add per step
            {"cvt_pk_u8", k_cvtpk, kChains},
            {"rndne", k_rndne, kChains},
            {"cvt_pk_fp8", k_cvt_fp8, kChains},              // instructions (two values each)
            {"cvt_2xpk16_fp6", k_cvt_fp6, 4}};               // instructions (32 values each)
  for (auto& v : vk) {
    RateCtx c{v.k, out, 4000, blocks};
    const float ms = time_ms(launch_rate, &c, 3);
    const double lane_ops = (double)blocks * 256 * c.iters * v.per_iter;
    printf(", \"%s_G_per_s\": %.1f", v.name, lane_ops / (ms * 1e-3) / 1e9);
  }
  {
    RateCtx c{k_fma64, out, 4000, blocks};
    const float ms = time_ms(launch_rate, &c, 3);
    const double lane_ops = (double)blocks * 256 * c.iters * kChains;
    printf(", \"fma64_G_per_s\": %.1f", lane_ops / (ms * 1e-3) / 1e9);
  }
  {
    RateCtx c{k_lds, out, 4000, blocks};
    const float ms = time_ms(launch_rate, &c, 3);
    const double bytes = (double)blocks * 256 * c.iters * 8 * 16;
    printf(", \"lds_read_b128_TBps\": %.2f", bytes / (ms * 1e-3) / 1e12);
  }
  {
    RateCtx c{k_mfma_i8, out, 2000, blocks};
    const float ms = time_ms(launch_rate, &c, 3);
    const double ops = (double)blocks * 4 * c.iters * 4 * 65536.0;
    printf(", \"mfma_i8_32x32x32_TOPS\": %.1f", ops / (ms * 1e-3) / 1e12);
  }
  {
    RateCtx c{k_mfma_f16, out, 2000, blocks};
    const float ms = time_ms(launch_rate, &c, 3);
    const double ops = (double)blocks * 4 * c.iters * 4 * 32768.0;
    printf(", \"mfma_f16_32x32x16_TFLOPS\": %.1f", ops / (ms * 1e-3) / 1e12);
  }
  for (int vpm : {4, 8, 16}) {
    MixCtx c{out, 2000, blocks, vpm};
    const float ms = time_ms(launch_mix, &c, 3);
    const double ops = (double)blocks * 2 * c.iters * 4 * 65536.0;   // two MFMA waves per block
    printf(", \"mix_i8_with_%d_fma_per_mfma_TOPS\": %.1f", vpm, ops / (ms * 1e-3) / 1e12);
  }
  {
    // same-wave mix, in SIMD clocks per step at 2.4 GHz (one step of one wave;
    // 8 waves per SIMD share the SIMD)
    const double steps = (double)blocks * 4 / (cus * 4) * 2000 * 4;   // per SIMD
    void (*ks[4])(float*, int) = {k_mix_same<0>, k_mix_same<4>, k_mix_same<8>, k_mix_same<16>};
    const int ns[4] = {0, 4, 8, 16};
    for (int q = 0; q < 4; ++q) {
      RateCtx c{ks[q], out, 2000, blocks};
      const float ms = time_ms(launch_rate, &c, 3);
      printf(", \"same_wave_i8_mfma_plus_%d_fma_clocks_per_step\": %.1f", ns[q],
             ms * 1e-3 * 2.4e9 / steps);
    }
  }
  {
    const double steps_per_mfma = 65536.0 * 2;   // ops of one 32x32x64 MFMA
    void (*ks[3])(float*, int) = {k_mfma_f8f6f4<0, 0>, k_mfma_f8f6f4<0, 2>, k_mfma_f8f6f4<2, 2>};
    const char* nm[3] = {"fp8_fp8", "fp8_fp6", "fp6_fp6"};
    for (int q = 0; q < 3; ++q) {
      RateCtx c{ks[q], out, 1000, blocks};
      const float ms = time_ms(launch_rate, &c, 3);
      const double ops = (double)blocks * 4 * c.iters * 4 * steps_per_mfma;
      printf(", \"mfma_%s_32x32x64_TOPS\": %.1f", nm[q], ops / (ms * 1e-3) / 1e12);
    }
  }
  {
    // FP8 MFMA waves beside vector waves: ms for both, MFMA only, vector only
    struct F8Ctx {
      void (*k)(float*, int, int, int);
      float* out;
      int iters, blocks, vpm, mode;
    };
    auto launch_f8 = [](void* p) {
      F8Ctx* c = (F8Ctx*)p;
      hipLaunchKernelGGL(c->k, dim3(c->blocks), dim3(256), 0, 0, c->out, c->iters, c->vpm, c->mode);
    };
    void (*ks[4])(float*, int, int, int) = {k_mix_f8<0>, k_mix_f8<1>, k_mix_f8<2>, k_mix_f8<3>};
    const char* on[4] = {"fma", "exp", "max3", "mul"};
    for (int op = 0; op < 4; ++op)
      for (int vpm : {8, 16}) {
        float t[3];
        for (int mode = 0; mode < 3; ++mode) {
          F8Ctx c{ks[op], out, 1000, blocks, vpm, mode};
          t[mode] = time_ms(launch_f8, &c, 3);
        }
        printf(", \"f8mfma_with_%d_%s_ms_both_mfma_valu\": [%.4f, %.4f, %.4f]", vpm, on[op], t[0],
               t[1], t[2]);
      }
  }
  {
    // exponential waves and FMA waves side by side (3 FMAs per exponential in
    // the FMA waves), ms for both kinds and for each alone
    struct ModeCtx {
      float* out;
      int iters, blocks, mode;
    };
    auto launch_mode = [](void* p) {
      ModeCtx* c = (ModeCtx*)p;
      hipLaunchKernelGGL(k_exp_fma_waves, dim3(c->blocks), dim3(256), 0, 0, c->out, c->iters,
                         c->mode);
    };
    const char* nm[3] = {"both", "exp_only", "fma_only"};
    for (int mode = 0; mode < 3; ++mode) {
      ModeCtx c{out, 2000, blocks, mode};
      const float ms = time_ms(launch_mode, &c, 3);
      printf(", \"exp_and_fma_waves_%s_ms\": %.4f", nm[mode], ms);
    }
  }
  {
    // one v_exp_f32 plus N independent v_fma_f32 per step, SIMD clocks per step
    const double steps = (double)blocks * 4 / (cus * 4) * 4000 * kChains;   // per SIMD
    void (*ks[5])(float*, int) = {k_exp_mix<0>, k_exp_mix<1>, k_exp_mix<2>, k_exp_mix<3>,
                                  k_exp_mix<4>};
    for (int q = 0; q < 5; ++q) {
      RateCtx c{ks[q], out, 4000, blocks};
      const float ms = time_ms(launch_rate, &c, 3);
      printf(", \"same_wave_exp_plus_%d_fma_clocks_per_step\": %.2f", q,
             ms * 1e-3 * 2.4e9 / steps);
    }
  }
  printf("}\n");
  CK(hipFree(out));
  return 0;
}

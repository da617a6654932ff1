// Host side of librotattn.so: argument validation, buffer layout, the
// host-computed constants (RoPE tables, P-code thresholds, kappa) and the
// launch sequence of the C ABI declared in include/rotattn.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "rotattn_internal.h"

using namespace rotattn;

// Device scratch of rotattn_fp16_fwd_noalloc: staged Q', K' and V^T tiles of
// as many heads as fit, a chunk of heads at a time.  Each GPU the library
// runs on holds its own copy for the life of the process.  In host code the
// name stands for a host-side shadow, never the device address: the address
// is taken once per device with hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[ROTATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kRotBytes = kRotTabOffset;   // rotation scratch before the tables

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// The library scratch of a rotattn_prepared: the rotation (fp64 and the
// prologue's fp32 fragments), then the RoPE tables as (cos, sin) pairs, one
// 8-byte pair per (position, channel pair) of each axis.
size_t scratch_bytes(const rotattn_shape* s) {
  const size_t pairs = (size_t)s->grid_t * (s->d_t / 2) + (size_t)s->grid_h * (s->d_h / 2) +
                       (size_t)s->grid_w * (s->d_w / 2);
  return kRotBytes + align_up(pairs * 8);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int nblocks(const rotattn_shape* s) { return (s->N + kBlock - 1) / kBlock; }

// Head bitmask from a per-head byte mask: bit set where (mask[i] != 0) == want.
HeadBits make_bits(const uint8_t* mask, int BH, bool want, bool null_means_all, int* count) {
  HeadBits hb;
  memset(&hb, 0, sizeof(hb));
  int c = 0;
  for (int i = 0; i < BH; ++i) {
    const bool on = mask ? ((mask[i] != 0) == want) : null_means_all;
    if (on) {
      hb.w[i >> 5] |= 1u << (i & 31);
      ++c;
    }
  }
  if (count) *count = c;
  return hb;
}

float log2_15_f() { return (float)log2l(15.0L); }

}  // namespace

extern "C" {

int rotattn_validate(const rotattn_shape* s) {
  if (!s) return ROTATTN_E_NULL;
  if (s->B <= 0 || s->H <= 0 || s->N <= 0 || s->D <= 0 || s->grid_t <= 0 || s->grid_h <= 0 ||
      s->grid_w <= 0 || s->d_t <= 0 || s->d_h <= 0 || s->d_w <= 0)
    return ROTATTN_E_SHAPE;
  if ((int64_t)s->grid_t * s->grid_h * s->grid_w != (int64_t)s->N) return ROTATTN_E_SHAPE;
  if (s->d_t + s->d_h + s->d_w != s->D) return ROTATTN_E_SHAPE;
  if ((s->d_t | s->d_h | s->d_w) & 1) return ROTATTN_E_SHAPE;
  const bool split_ok = (s->D == 128 && s->d_t == 44 && s->d_h == 42 && s->d_w == 42) ||
                        (s->D == 64 && s->d_t == 24 && s->d_h == 20 && s->d_w == 20);
  if (!split_ok) return ROTATTN_E_UNSUPPORTED;
  if ((int64_t)s->B * s->H > ROTATTN_MAX_HEADS) return ROTATTN_E_UNSUPPORTED;
  if (s->N > (1 << 26)) return ROTATTN_E_UNSUPPORTED;   // keeps every index below 2^31 per head
  return ROTATTN_OK;
}

const char* rotattn_strerror(int status) {
  switch (status) {
    case ROTATTN_OK: return "ok";
    case ROTATTN_E_NULL: return "null pointer argument";
    case ROTATTN_E_SHAPE: return "inconsistent shape";
    case ROTATTN_E_UNSUPPORTED: return "unsupported head dimension, RoPE split or head count";
    case ROTATTN_E_WORKSPACE: return "workspace too small";
    case ROTATTN_E_ALIGN: return "device pointer not 16-byte aligned";
    case ROTATTN_E_HIP: return "HIP launch or runtime error";
    case ROTATTN_E_ARG: return "argument out of range";
    case ROTATTN_E_SCRATCH: return "one head exceeds the library's static scratch";
    default: return "unknown status";
  }
}

int rotattn_rope_tables_phase_host(const rotattn_shape* s, double base, const double* phase_t,
                                   const double* phase_h, const double* phase_w, float* cos_t,
                                   float* sin_t, float* cos_h, float* sin_h, float* cos_w,
                                   float* sin_w) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!cos_t || !sin_t || !cos_h || !sin_h || !cos_w || !sin_w) return ROTATTN_E_NULL;
  if (!(base > 1.0)) return ROTATTN_E_ARG;
  const int ext[3] = {s->grid_t, s->grid_h, s->grid_w};
  const int wid[3] = {s->d_t, s->d_h, s->d_w};
  const double* ph[3] = {phase_t, phase_h, phase_w};
  float* cs[3] = {cos_t, cos_h, cos_w};
  float* sn[3] = {sin_t, sin_h, sin_w};
  for (int a = 0; a < 3; ++a) {
    const int half = wid[a] / 2;
    for (int j = 0; j < half; ++j) {
      const long double theta = powl((long double)base, -2.0L * j / (long double)wid[a]);
      const long double phi = ph[a] ? (long double)ph[a][j] : 0.0L;
      if (ph[a] && !isfinite(ph[a][j])) return ROTATTN_E_ARG;
      for (int p = 0; p < ext[a]; ++p) {
        const long double ang = (long double)p * theta + phi;
        cs[a][p * half + j] = (float)cosl(ang);
        sn[a][p * half + j] = (float)sinl(ang);
      }
    }
  }
  return ROTATTN_OK;
}

int rotattn_rope_tables_host(const rotattn_shape* s, double base, float* cos_t, float* sin_t,
                             float* cos_h, float* sin_h, float* cos_w, float* sin_w) {
  return rotattn_rope_tables_phase_host(s, base, nullptr, nullptr, nullptr, cos_t, sin_t, cos_h,
                                        sin_h, cos_w, sin_w);
}

int rotattn_pcode_thresholds_host(float tau[15]) {
  if (!tau) return ROTATTN_E_NULL;
  for (int k = 1; k <= 15; ++k) {
    const long double v = log2l((long double)(2 * k - 1) / 30.0L);
    float f = (float)v;
    while ((long double)f < v) f = nextafterf(f, INFINITY);
    while ((long double)nextafterf(f, -INFINITY) >= v) f = nextafterf(f, -INFINITY);
    tau[k - 1] = f;
  }
  return ROTATTN_OK;
}

float rotattn_kappa_host(int32_t D) {
  if (D <= 0) return 0.0f;
  return (float)(1.0L / logl(2.0L) / sqrtl((long double)D));
}

static bool valid_layout(int layout) {
  return layout == ROTATTN_LAYOUT_PACKED || layout == ROTATTN_LAYOUT_FP8 ||
         layout == ROTATTN_LAYOUT_FP6;
}

// FP8 and FP6: one byte per code (FP6 groups of 32 codes in 24 bytes + 8 pad)
static bool byte_layout(int layout) {
  return layout == ROTATTN_LAYOUT_FP8 || layout == ROTATTN_LAYOUT_FP6;
}

size_t rotattn_prepared_bytes_layout(const rotattn_shape* s, int with_rope, int layout) {
  if (rotattn_validate(s) != ROTATTN_OK) return 0;
  if (!valid_layout(layout)) return 0;
  const size_t BH = (size_t)s->B * s->H, NB = nblocks(s), D = s->D;
  const size_t per_code = byte_layout(layout) ? 2 : 1;   // half-bytes per code
  const size_t packed = align_up(BH * NB * kBlock * D * per_code / 2);
  const size_t scales = align_up(BH * NB * sizeof(float));
  // fallback buffers: q_rope, k_rope, v_t, each [B*H][N_pad][D] fp16
  const size_t rope = with_rope ? align_up(BH * NB * kBlock * D * 2) : 0;
  return 3 * packed + 3 * scales + scratch_bytes(s) + 3 * rope;
}

int rotattn_prepared_carve(const rotattn_shape* s, void* base, size_t bytes, int with_rope,
                           int layout, rotattn_prepared* out) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!base || !out) return ROTATTN_E_NULL;
  if (!valid_layout(layout)) return ROTATTN_E_ARG;
  if (((uintptr_t)base & (kAlign - 1)) != 0) return ROTATTN_E_ALIGN;
  if (bytes < rotattn_prepared_bytes_layout(s, with_rope, layout)) return ROTATTN_E_WORKSPACE;
  const size_t BH = (size_t)s->B * s->H, NB = nblocks(s), D = s->D;
  const size_t per_code = byte_layout(layout) ? 2 : 1;
  const size_t packed = align_up(BH * NB * kBlock * D * per_code / 2);
  const size_t scales = align_up(BH * NB * sizeof(float));
  const size_t rope = align_up(BH * NB * kBlock * D * 2);
  uint8_t* p = (uint8_t*)base;
  out->layout = layout;
  out->q4 = p; p += packed;
  out->k4 = p; p += packed;
  out->v4 = p; p += packed;
  out->q_scale_l2 = (float*)p; p += scales;
  out->k_scale = (float*)p; p += scales;
  out->v_scale = (float*)p; p += scales;
  out->rot64 = (double*)p; p += scratch_bytes(s);
  if (with_rope) {
    out->q_rope = (uint16_t*)p; p += rope;
    out->k_rope = (uint16_t*)p; p += rope;
    out->v_t = (uint16_t*)p; p += rope;
  } else {
    out->q_rope = nullptr;
    out->k_rope = nullptr;
    out->v_t = nullptr;
  }
  return ROTATTN_OK;
}

size_t rotattn_prepared_bytes(const rotattn_shape* s) {
  return rotattn_prepared_bytes_layout(s, 1, ROTATTN_LAYOUT_FP6);
}

// Strides of a tensor, contiguous [B][H][N][D] when st is NULL.  Every stride
// must keep 16-byte rows (a multiple of 8 elements), and rows of one head must
// not overlap (token >= D).
static int resolve_strides(const rotattn_shape* s, const rotattn_strides* st, Strides* out) {
  if (!st) {
    out->batch = (int64_t)s->H * s->N * s->D;
    out->head = (int64_t)s->N * s->D;
    out->token = s->D;
    return ROTATTN_OK;
  }
  if (st->batch < 0 || st->head < 0 || st->token < s->D) return ROTATTN_E_ARG;
  if (st->batch % 8 || st->head % 8 || st->token % 8) return ROTATTN_E_ALIGN;
  out->batch = st->batch;
  out->head = st->head;
  out->token = st->token;
  return ROTATTN_OK;
}

int rotattn_prepare_qkv(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const rotattn_rope_rot* rr,
                        const uint8_t* fallback_mask_host, const rotattn_prepared* out,
                        hipStream_t stream) {
  return rotattn_prepare_qkv_strided(s, q, k, v, nullptr, rr, fallback_mask_host, out, stream);
}

}  // extern "C"

namespace {

// The prologue's checks of its tables and output buffers, nothing enqueued.
int check_prepare_out(const rotattn_shape* s, const rotattn_rope_rot* rr,
                      const uint8_t* fallback_mask_host, const rotattn_prepared* out) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!rr || !out) return ROTATTN_E_NULL;
  if (!rr->cos_t || !rr->sin_t || !rr->cos_h || !rr->sin_h || !rr->cos_w || !rr->sin_w)
    return ROTATTN_E_NULL;
  // all three rotation matrices, or none (rotation merged into the tables)
  const int n_rot = (rr->rot_t != nullptr) + (rr->rot_h != nullptr) + (rr->rot_w != nullptr);
  if (n_rot != 0 && n_rot != 3) return ROTATTN_E_NULL;
  const int BH = s->B * s->H;
  if (!valid_layout(out->layout)) return ROTATTN_E_ARG;
  int n_fb = 0;
  make_bits(fallback_mask_host, BH, true, false, &n_fb);
  if (n_fb < BH) {
    if (!out->q4 || !out->k4 || !out->v4 || !out->q_scale_l2 || !out->k_scale || !out->v_scale ||
        !out->rot64)
      return ROTATTN_E_NULL;
    if (!aligned16(out->q4) || !aligned16(out->k4) || !aligned16(out->v4)) return ROTATTN_E_ALIGN;
  }
  if (n_fb > 0) {
    if (!out->q_rope || !out->k_rope || !out->v_t) return ROTATTN_E_NULL;
    if (!aligned16(out->q_rope) || !aligned16(out->k_rope) || !aligned16(out->v_t))
      return ROTATTN_E_ALIGN;
  }
  return ROTATTN_OK;
}

// Every argument check of the prologue, nothing enqueued.
int check_prepare(const rotattn_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const rotattn_strides* qkv_strides, const rotattn_rope_rot* rr,
                  const uint8_t* fallback_mask_host, const rotattn_prepared* out, Strides* in) {
  const int st = check_prepare_out(s, rr, fallback_mask_host, out);
  if (st != ROTATTN_OK) return st;
  if (!q || !k || !v) return ROTATTN_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ROTATTN_E_ALIGN;
  return resolve_strides(s, qkv_strides, in);
}

// The prologue's arguments apart from its inputs (q, k, v, in left null), with
// the rotation converted to fp64 on the stream when a head needs it.
int prologue_args(const rotattn_shape* s, const rotattn_rope_rot* rr,
                  const uint8_t* fallback_mask_host, const rotattn_prepared* out,
                  hipStream_t stream, PrologueArgs* pa) {
  const bool rot = rr->rot_t != nullptr;
  const int BH = s->B * s->H;
  int n_fb = 0;
  const HeadBits fb = make_bits(fallback_mask_host, BH, true, false, &n_fb);
  if (rot && n_fb < BH &&
      launch_rot_to_f64(rr->rot_t, rr->rot_h, rr->rot_w, s->d_t, s->d_h, out->rot64, stream) !=
          hipSuccess)
    return ROTATTN_E_HIP;
  float* tabs = (float*)((uint8_t*)out->rot64 + kRotTabOffset);
  const int np_t = s->grid_t * (s->d_t / 2), np_h = s->grid_h * (s->d_h / 2);
  const int np_w = s->grid_w * (s->d_w / 2);
  if (n_fb < BH && launch_rope_pairs(rr, np_t, np_h, np_w, tabs, stream) != hipSuccess)
    return ROTATTN_E_HIP;
  PrologueArgs& a = *pa;
  a.cs_t = tabs;
  a.cs_h = tabs + 2 * np_t;
  a.cs_w = tabs + 2 * (np_t + np_h);
  a.q = a.k = a.v = nullptr;
  a.in = Strides{};
  a.H = s->H;
  a.cos_t = rr->cos_t; a.sin_t = rr->sin_t;
  a.cos_h = rr->cos_h; a.sin_h = rr->sin_h;
  a.cos_w = rr->cos_w; a.sin_w = rr->sin_w;
  a.rot64 = out->rot64;
  a.q4 = out->q4; a.k4 = out->k4; a.v4 = out->v4;
  a.q_scale_l2 = out->q_scale_l2; a.k_scale = out->k_scale; a.v_scale = out->v_scale;
  a.q_rope = out->q_rope; a.k_rope = out->k_rope; a.v_t = out->v_t;
  a.N = s->N;
  a.NB = nblocks(s);
  a.grid_h = s->grid_h;
  a.grid_w = s->grid_w;
  a.kappa = rotattn_kappa_host(s->D);
  a.fallback = fb;
  return ROTATTN_OK;
}

int launch_prepare(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const Strides& in, const rotattn_rope_rot* rr,
                   const uint8_t* fallback_mask_host, const rotattn_prepared* out,
                   hipStream_t stream) {
  PrologueArgs a;
  const int r = prologue_args(s, rr, fallback_mask_host, out, stream, &a);
  if (r != ROTATTN_OK) return r;
  a.q = q; a.k = k; a.v = v;
  a.in = in;
  return launch_prologue(s->D, s->d_t, s->B * s->H, out->layout, rr->rot_t != nullptr, a,
                         stream) == hipSuccess
             ? ROTATTN_OK
             : ROTATTN_E_HIP;
}

// Every argument check of the fused QKV projection + prologue, nothing enqueued.
int check_qkv_proj(const rotattn_shape* s, const uint16_t* x, int64_t x_batch, int64_t x_token,
                   int32_t C, const uint16_t* w, const rotattn_rope_rot* rr,
                   const uint8_t* fallback_mask_host, const rotattn_prepared* out,
                   const uint16_t* qkv_out) {
  const int st = check_prepare_out(s, rr, fallback_mask_host, out);
  if (st != ROTATTN_OK) return st;
  if (!x || !w) return ROTATTN_E_NULL;
  if (s->D != 128 || s->d_t != 44) return ROTATTN_E_UNSUPPORTED;
  // a work-group's row offsets within its 128 rows are 32-bit byte offsets
  if (C < 64 || C % 64 != 0 || x_token < C || x_token > (1 << 24) || x_batch < 0)
    return ROTATTN_E_ARG;
  if (s->B > 1 && x_batch < (int64_t)s->N * x_token) return ROTATTN_E_ARG;
  if (!aligned16(x) || !aligned16(w) || (qkv_out && !aligned16(qkv_out)) || x_token % 8 != 0 ||
      x_batch % 8 != 0)
    return ROTATTN_E_ALIGN;
  return ROTATTN_OK;
}

// Every argument check of the INT4 attention, nothing enqueued.
int check_int4(const rotattn_shape* s, const rotattn_prepared* p, uint16_t* o,
               const rotattn_strides* o_strides, const rotattn_int4_opts* opts,
               const rotattn_debug* dbg, Strides* os) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!p || !o) return ROTATTN_E_NULL;
  const int sr = resolve_strides(s, o_strides, os);
  if (sr != ROTATTN_OK) return sr;
  if (!p->q4 || !p->k4 || !p->v4 || !p->q_scale_l2 || !p->k_scale || !p->v_scale)
    return ROTATTN_E_NULL;
  if (!aligned16(p->q4) || !aligned16(p->k4) || !aligned16(p->v4) || !aligned16(o))
    return ROTATTN_E_ALIGN;
  if (!valid_layout(p->layout)) return ROTATTN_E_ARG;
  const int norm = opts ? opts->normalizer : ROTATTN_NORM_EXP;
  if (norm != ROTATTN_NORM_EXP && norm != ROTATTN_NORM_CODES) return ROTATTN_E_ARG;
  if (norm == ROTATTN_NORM_CODES && !byte_layout(p->layout)) return ROTATTN_E_UNSUPPORTED;
  if (dbg) {
    if (!dbg->s_int || !dbg->p_code || !dbg->pv_int || !dbg->m_final || !dbg->l_final)
      return ROTATTN_E_NULL;
    if (dbg->b < 0 || dbg->b >= s->B || dbg->h < 0 || dbg->h >= s->H || dbg->q_block < 0 ||
        dbg->q_block >= nblocks(s))
      return ROTATTN_E_ARG;
  }
  return ROTATTN_OK;
}

int launch_int4_all(const rotattn_shape* s, const rotattn_prepared* p,
                    const uint8_t* fallback_mask_host, uint16_t* o, const Strides& os,
                    const rotattn_int4_opts* opts, const rotattn_debug* dbg, hipStream_t stream) {
  const bool f8 = byte_layout(p->layout);
  const int norm = opts ? opts->normalizer : ROTATTN_NORM_EXP;
  const int BH = s->B * s->H;
  Int4Debug d{};
  if (dbg) {
    d.s_int = dbg->s_int;
    d.p_code = dbg->p_code;
    d.pv_int = dbg->pv_int;
    d.m_final = dbg->m_final;
    d.l_final = dbg->l_final;
    d.bh = dbg->b * s->H + dbg->h;
    d.q_block = dbg->q_block;
  }
  int n_run = 0;
  Int4Args a;
  a.run = make_bits(fallback_mask_host, BH, false, true, &n_run);
  a.q4 = p->q4; a.k4 = p->k4; a.v4 = p->v4;
  a.q_scale_l2 = p->q_scale_l2; a.k_scale = p->k_scale; a.v_scale = p->v_scale;
  a.o = o;
  a.os = os;
  a.H = s->H;
  a.N = s->N;
  a.NB = nblocks(s);
  a.log2_15 = log2_15_f();
  a.code_sum = norm == ROTATTN_NORM_CODES;
  a.f6 = p->layout == ROTATTN_LAYOUT_FP6;
  rotattn_pcode_thresholds_host(a.tau);
  auto launch = f8 ? launch_int4_f8 : launch_int4;
  if (n_run > 0 && launch(s->D, BH, a, nullptr, stream) != hipSuccess) return ROTATTN_E_HIP;
  if (dbg && launch(s->D, BH, a, &d, stream) != hipSuccess) return ROTATTN_E_HIP;
  return ROTATTN_OK;
}

// Every argument check of the FP16 attention on prepared buffers, nothing enqueued.
int check_fp16_prepared(const rotattn_shape* s, const rotattn_prepared* p, uint16_t* o,
                        const rotattn_strides* o_strides, Strides* os) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!p || !o) return ROTATTN_E_NULL;
  const int sr = resolve_strides(s, o_strides, os);
  if (sr != ROTATTN_OK) return sr;
  if (!p->q_rope || !p->k_rope || !p->v_t) return ROTATTN_E_NULL;
  if (!aligned16(p->q_rope) || !aligned16(p->k_rope) || !aligned16(p->v_t) || !aligned16(o))
    return ROTATTN_E_ALIGN;
  return ROTATTN_OK;
}

// FP16 attention over the selected global heads bh0 .. bh0 + nbh - 1 whose
// padded Q', K' and V^T tiles start at q, k, v_t.
int launch_fp16_heads(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v_t, const HeadBits& run, int bh0, int nbh, uint16_t* o,
                      const Strides& os, hipStream_t stream) {
  Fp16Args a;
  a.run = run;
  a.q = q; a.k = k; a.v_t = v_t; a.o = o;
  a.os = os;
  a.H = s->H;
  a.N = s->N;
  a.NB = nblocks(s);
  a.kappa = rotattn_kappa_host(s->D);
  a.bh0 = bh0;
  return launch_fp16(s->D, nbh, a, stream) == hipSuccess ? ROTATTN_OK : ROTATTN_E_HIP;
}

// Bytes of one head's staged fp16 buffers (padded Q', K', V^T tiles).
size_t fp16_head_bytes(const rotattn_shape* s) {
  return (size_t)nblocks(s) * kBlock * s->D * 2;
}

// Stage heads bh0 .. bh0 + nbh - 1 (selected ones only) into q_pad, k_pad,
// v_t and run the FP16 attention on them.
int stage_and_run_fp16(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const Strides& in, const HeadBits& run, int bh0,
                       int nbh, uint16_t* q_pad, uint16_t* k_pad, uint16_t* v_t, uint16_t* o,
                       const Strides& os, hipStream_t stream) {
  StageArgs g;
  g.q = q; g.k = k; g.v = v;
  g.in = in;
  g.H = s->H;
  g.N = s->N;
  g.NB = nblocks(s);
  g.q_pad = q_pad; g.k_pad = k_pad; g.v_t = v_t;
  g.run = run;
  g.bh0 = bh0;
  if (launch_stage_fp16(s->D, nbh, g, stream) != hipSuccess) return ROTATTN_E_HIP;
  return launch_fp16_heads(s, q_pad, k_pad, v_t, run, bh0, nbh, o, os, stream);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current); NULL if the lookup fails.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int rotattn_prepare_qkv_strided(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const rotattn_strides* qkv_strides,
                                const rotattn_rope_rot* rr, const uint8_t* fallback_mask_host,
                                const rotattn_prepared* out, hipStream_t stream) {
  Strides in;
  const int st = check_prepare(s, q, k, v, qkv_strides, rr, fallback_mask_host, out, &in);
  if (st != ROTATTN_OK) return st;
  return launch_prepare(s, q, k, v, in, rr, fallback_mask_host, out, stream);
}

int rotattn_qkv_proj_prepare(const rotattn_shape* s, const uint16_t* x, int64_t x_batch,
                             int64_t x_token, int32_t C, const uint16_t* w, const uint16_t* bias,
                             const rotattn_rope_rot* rr, const uint8_t* fallback_mask_host,
                             const rotattn_prepared* out, uint16_t* qkv_out,
                             hipStream_t stream) {
  const int st = check_qkv_proj(s, x, x_batch, x_token, C, w, rr, fallback_mask_host, out,
                                qkv_out);
  if (st != ROTATTN_OK) return st;
  QkvProjArgs a;
  const int r = prologue_args(s, rr, fallback_mask_host, out, stream, &a.p);
  if (r != ROTATTN_OK) return r;
  a.x = x;
  a.x_batch = x_batch;
  a.x_token = x_token;
  a.w = w;
  a.bias = bias;
  a.qkv_out = qkv_out;
  a.C = C;
  a.B = s->B;
  a.SBT = a.SHT = a.last_block_only = 0;   // set per launch
  return launch_qkv_proj(s->D, s->d_t, out->layout, rr->rot_t != nullptr, a, stream) == hipSuccess
             ? ROTATTN_OK
             : ROTATTN_E_HIP;
}

int rotattn_int4_fwd(const rotattn_shape* s, const rotattn_prepared* p,
                     const uint8_t* fallback_mask_host, uint16_t* o, const rotattn_debug* dbg,
                     hipStream_t stream) {
  return rotattn_int4_fwd_strided(s, p, fallback_mask_host, o, nullptr, nullptr, dbg, stream);
}

int rotattn_int4_fwd_strided(const rotattn_shape* s, const rotattn_prepared* p,
                             const uint8_t* fallback_mask_host, uint16_t* o,
                             const rotattn_strides* o_strides, const rotattn_int4_opts* opts,
                             const rotattn_debug* dbg, hipStream_t stream) {
  Strides os;
  const int st = check_int4(s, p, o, o_strides, opts, dbg, &os);
  if (st != ROTATTN_OK) return st;
  return launch_int4_all(s, p, fallback_mask_host, o, os, opts, dbg, stream);
}

int rotattn_fp16_fwd_prepared(const rotattn_shape* s, const rotattn_prepared* p,
                              const uint8_t* head_select_host, uint16_t* o, hipStream_t stream) {
  return rotattn_fp16_fwd_prepared_strided(s, p, head_select_host, o, nullptr, stream);
}

int rotattn_fp16_fwd_prepared_strided(const rotattn_shape* s, const rotattn_prepared* p,
                                      const uint8_t* head_select_host, uint16_t* o,
                                      const rotattn_strides* o_strides, hipStream_t stream) {
  Strides os;
  const int st = check_fp16_prepared(s, p, o, o_strides, &os);
  if (st != ROTATTN_OK) return st;
  int n_run = 0;
  const HeadBits run = make_bits(head_select_host, s->B * s->H, true, true, &n_run);
  if (n_run == 0) return ROTATTN_OK;
  return launch_fp16_heads(s, p->q_rope, p->k_rope, p->v_t, run, 0, s->B * s->H, o, os, stream);
}

size_t rotattn_fp16_workspace_bytes(const rotattn_shape* s) {
  if (rotattn_validate(s) != ROTATTN_OK) return 0;
  return 3 * align_up((size_t)s->B * s->H * fp16_head_bytes(s));
}

int rotattn_fp16_fwd(const rotattn_shape* s, const uint16_t* q_rope, const uint16_t* k_rope,
                     const uint16_t* v, const uint8_t* head_select_host, void* workspace,
                     size_t workspace_bytes, uint16_t* o, hipStream_t stream) {
  return rotattn_fp16_fwd_strided(s, q_rope, k_rope, v, nullptr, head_select_host, workspace,
                                  workspace_bytes, o, nullptr, stream);
}

int rotattn_fp16_fwd_strided(const rotattn_shape* s, const uint16_t* q_rope,
                             const uint16_t* k_rope, const uint16_t* v,
                             const rotattn_strides* qkv_strides, const uint8_t* head_select_host,
                             void* workspace, size_t workspace_bytes, uint16_t* o,
                             const rotattn_strides* o_strides, hipStream_t stream) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!q_rope || !k_rope || !v || !workspace || !o) return ROTATTN_E_NULL;
  if (!aligned16(q_rope) || !aligned16(k_rope) || !aligned16(v) || !aligned16(o) ||
      !aligned16(workspace))
    return ROTATTN_E_ALIGN;
  Strides in, os;
  int r = resolve_strides(s, qkv_strides, &in);
  if (r != ROTATTN_OK) return r;
  r = resolve_strides(s, o_strides, &os);
  if (r != ROTATTN_OK) return r;
  if (workspace_bytes < rotattn_fp16_workspace_bytes(s)) return ROTATTN_E_WORKSPACE;
  const int BH = s->B * s->H;
  int n_run = 0;
  const HeadBits run = make_bits(head_select_host, BH, true, true, &n_run);
  if (n_run == 0) return ROTATTN_OK;
  const size_t part = align_up((size_t)BH * fp16_head_bytes(s));
  uint8_t* w = (uint8_t*)workspace;
  return stage_and_run_fp16(s, q_rope, k_rope, v, in, run, 0, BH, (uint16_t*)w,
                            (uint16_t*)(w + part), (uint16_t*)(w + 2 * part), o, os, stream);
}

int rotattn_fp16_fwd_noalloc(const rotattn_shape* s, const uint16_t* q_rope,
                             const uint16_t* k_rope, const uint16_t* v,
                             const uint8_t* head_select_host, uint16_t* o, hipStream_t stream) {
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!q_rope || !k_rope || !v || !o) return ROTATTN_E_NULL;
  if (!aligned16(q_rope) || !aligned16(k_rope) || !aligned16(v) || !aligned16(o))
    return ROTATTN_E_ALIGN;
  // three staged arrays per head, each part 256-byte aligned
  const size_t per_head = 3 * align_up(fp16_head_bytes(s));
  const int chunk = (int)(ROTATTN_NOALLOC_SCRATCH_BYTES / per_head);
  if (chunk < 1) return ROTATTN_E_SCRATCH;
  const int BH = s->B * s->H;
  int n_run = 0;
  const HeadBits run = make_bits(head_select_host, BH, true, true, &n_run);
  if (n_run == 0) return ROTATTN_OK;
  uint8_t* base = (uint8_t*)scratch_on_current_device();
  if (!base) return ROTATTN_E_HIP;
  Strides in, os;
  resolve_strides(s, nullptr, &in);
  resolve_strides(s, nullptr, &os);
  for (int bh0 = 0; bh0 < BH; bh0 += chunk) {
    const int nbh = BH - bh0 < chunk ? BH - bh0 : chunk;
    bool any = false;
    for (int i = bh0; i < bh0 + nbh; ++i) any = any || run.test(i);
    if (!any) continue;
    // the staging of this chunk follows the previous chunk's attention on the
    // same stream, so it never overwrites data still being read
    const size_t part = align_up((size_t)nbh * fp16_head_bytes(s));
    const int r = stage_and_run_fp16(s, q_rope, k_rope, v, in, run, bh0, nbh, (uint16_t*)base,
                                     (uint16_t*)(base + part), (uint16_t*)(base + 2 * part), o,
                                     os, stream);
    if (r != ROTATTN_OK) return r;
  }
  return ROTATTN_OK;
}

size_t rotattn_workspace_bytes(const rotattn_shape* s) {
  return rotattn_prepared_bytes_layout(s, 1, ROTATTN_LAYOUT_FP6);
}

int rotattn_mixed_fwd(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const rotattn_rope_rot* rr,
                      const uint8_t* fallback_mask_host, void* workspace, size_t workspace_bytes,
                      uint16_t* o, hipStream_t stream) {
  return rotattn_mixed_fwd_strided(s, q, k, v, nullptr, rr, fallback_mask_host, workspace,
                                   workspace_bytes, o, nullptr, stream);
}

int rotattn_mixed_fwd_strided(const rotattn_shape* s, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const rotattn_strides* qkv_strides,
                              const rotattn_rope_rot* rr, const uint8_t* fallback_mask_host,
                              void* workspace, size_t workspace_bytes, uint16_t* o,
                              const rotattn_strides* o_strides, hipStream_t stream) {
  // every argument is checked before anything is enqueued
  const int st = rotattn_validate(s);
  if (st != ROTATTN_OK) return st;
  if (!q || !k || !v || !rr || !workspace || !o) return ROTATTN_E_NULL;
  rotattn_prepared p;
  int r = rotattn_prepared_carve(s, workspace, workspace_bytes, 1, ROTATTN_LAYOUT_FP6, &p);
  if (r != ROTATTN_OK) return r;
  Strides in, os;
  r = check_prepare(s, q, k, v, qkv_strides, rr, fallback_mask_host, &p, &in);
  if (r != ROTATTN_OK) return r;
  r = check_int4(s, &p, o, o_strides, nullptr, nullptr, &os);
  if (r != ROTATTN_OK) return r;
  r = check_fp16_prepared(s, &p, o, o_strides, &os);
  if (r != ROTATTN_OK) return r;
  r = launch_prepare(s, q, k, v, in, rr, fallback_mask_host, &p, stream);
  if (r != ROTATTN_OK) return r;
  r = launch_int4_all(s, &p, fallback_mask_host, o, os, nullptr, nullptr, stream);
  if (r != ROTATTN_OK) return r;
  int n_fb = 0;
  const HeadBits fb = make_bits(fallback_mask_host, s->B * s->H, true, false, &n_fb);
  if (n_fb > 0) r = launch_fp16_heads(s, p.q_rope, p.k_rope, p.v_t, fb, 0, s->B * s->H, o, os, stream);
  return r;
}

int rotattn_pcode_sweep(int layout, uint32_t mag_lo, uint32_t count, uint32_t* transitions,
                        uint32_t max_transitions, uint32_t* n_transitions, hipStream_t stream) {
  if (!transitions || !n_transitions) return ROTATTN_E_NULL;
  if (!valid_layout(layout)) return ROTATTN_E_ARG;
  if (count == 0 || (uint64_t)mag_lo + count > 0x7B800000ull) return ROTATTN_E_ARG;
  float tau[15];
  rotattn_pcode_thresholds_host(tau);
  return launch_pcode_sweep(byte_layout(layout), mag_lo, count, tau, log2_15_f(),
                            transitions, max_transitions, n_transitions, stream) == hipSuccess
             ? ROTATTN_OK
             : ROTATTN_E_HIP;
}

int rotattn_pcode_eval(int layout, const int32_t* I, uint32_t n, float c, float m, uint8_t* codes,
                       hipStream_t stream) {
  if (!I || !codes) return ROTATTN_E_NULL;
  if (!valid_layout(layout)) return ROTATTN_E_ARG;
  if (n == 0 || (n % 4096u) != 0) return ROTATTN_E_ARG;
  if (!(c >= 0.0f) || !isfinite(m)) return ROTATTN_E_ARG;
  float tau[15];
  rotattn_pcode_thresholds_host(tau);
  return launch_pcode_eval(byte_layout(layout), I, n, c, m, tau, log2_15_f(), codes,
                           stream) == hipSuccess
             ? ROTATTN_OK
             : ROTATTN_E_HIP;
}

}  // extern "C"

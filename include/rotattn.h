/*
 * rotattn.h -- C ABI of librotattn.so: RotateAttention's mixed-precision INT4
 * FlashAttention forward for DiT video models with 3D RoPE, on AMD MI355X
 * (gfx950).
 *
 * Source: "RotateAttention: RoPE-Aware Rotation and Range Rectification for
 * INT4 Quantized Attention in Video Generation", Abstract.  The abstract
 * states the problem as attention inside DiT video generators that use 3D
 * RoPE, computed by a quantized FlashAttention whose Q and K are rotated by
 * RoPE-aware orthogonal matrices, whose probabilities P = exp(S - max S) are
 * quantized to the full unsigned INT4 range with a fixed scale and zero point,
 * and with a selective FP16 fallback for accuracy-sensitive heads.  The entry
 * points below are the steps of that forward pass:
 *
 *   rotattn_prepare_qkv  3D RoPE + partition-wise rotation + per-block INT4
 *                        quantize and pack (RoPE'd fp16 Q/K for fallback heads)
 *   rotattn_int4_fwd     integer QK^T, online softmax, u4 P, integer P.V
 *   rotattn_fp16_fwd     FP16 FlashAttention for the fallback heads, on the
 *                        caller's RoPE'd fp16 Q'/K' and V
 *   rotattn_mixed_fwd    all of the above on one stream, routed by a head mask
 *
 * Conventions (every entry point):
 *  - Tensors are device pointers owned by the caller.  The library never
 *    allocates device memory, never synchronizes, and enqueues work only on
 *    the stream it is given.  fp16 tensors are IEEE binary16 bit patterns
 *    (uint16_t).  Device pointers must be 16-byte aligned.
 *  - Shapes: Q, K, V, O are [B][H][N][D] contiguous.  Token n sits at
 *    t = n / (Hg*Wg), h = (n / Wg) % Hg, w = n % Wg of the latent grid
 *    (T, Hg, Wg) = (grid_t, grid_h, grid_w), so N = T*Hg*Wg.  The head
 *    dimension D is split into RoPE partitions [d_t | d_h | d_w] in that
 *    order; inside a partition channels (2j, 2j+1) form one rotary pair.
 *  - Supported: D in {64, 128}, (d_t, d_h, d_w) = (24, 20, 20) for D = 64 and
 *    (44, 42, 42) for D = 128, B*H <= ROTATTN_MAX_HEADS.
 *  - Host-side arrays (masks) are read during the call and not kept.
 *  - Return value: ROTATTN_OK (0) or a negative rotattn_status.  Argument
 *    errors are reported before anything is enqueued; a launch error maps to
 *    ROTATTN_E_HIP.  Nothing throws across the ABI and there is no mutable
 *    global state, so calls are re-entrant.
 *  - Non-finite inputs are undefined behaviour (not checked).
 */
#ifndef ROTATTN_H
#define ROTATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROTATTN_BLOCK 128        /* quantization block == key tile, in tokens */
#define ROTATTN_MAX_HEADS 4096   /* B*H limit (head masks travel as kernel arguments) */
#define ROTATTN_P_LEVELS 15      /* u4 P: scale 1/15, zero point 0 */

typedef enum rotattn_status {
  ROTATTN_OK = 0,
  ROTATTN_E_NULL = -1,          /* a required pointer is NULL */
  ROTATTN_E_SHAPE = -2,         /* inconsistent shape (N != T*Hg*Wg, d_t+d_h+d_w != D, odd d_a, <= 0) */
  ROTATTN_E_UNSUPPORTED = -3,   /* D or RoPE split outside the supported set, too many heads */
  ROTATTN_E_WORKSPACE = -4,     /* workspace smaller than rotattn_workspace_bytes() */
  ROTATTN_E_ALIGN = -5,         /* a device pointer is not 16-byte aligned */
  ROTATTN_E_HIP = -6,           /* a HIP launch or runtime call failed */
  ROTATTN_E_ARG = -7,           /* another argument is out of range (debug q-block, sweep range) */
  ROTATTN_E_SCRATCH = -8        /* a head's staging exceeds ROTATTN_NOALLOC_SCRATCH_BYTES */
} rotattn_status;

/* Size of the library's static device scratch (rotattn_fp16_fwd_noalloc). */
#define ROTATTN_NOALLOC_SCRATCH_BYTES (256u << 20)

/* Problem shape. */
typedef struct rotattn_shape {
  int32_t B, H, N, D;
  int32_t grid_t, grid_h, grid_w;
  int32_t d_t, d_h, d_w;
} rotattn_shape;

/*
 * RoPE tables and rotation matrices (device, fp32, caller-owned).
 * cos_a/sin_a: [extent_a][d_a/2] with entry [p][j] = cos/sin(p * theta_{a,j}
 * + phi_{a,j}), theta_{a,j} = base^(-2j/d_a); rotattn_rope_tables_host()
 * fills them with phi = 0, rotattn_rope_tables_phase_host() with phases.
 * rot_a: [d_a][d_a] row-major orthogonal matrix, row = output channel; the
 * same matrices apply to Q and K of every head (RoPE-aware rotation inside
 * each RoPE partition, applied after RoPE; RotateAttention page, Abstract).
 * rot_t, rot_h and rot_w may all be NULL: then no dense rotation is applied
 * (z = the RoPE'd values), which is the form of a rotation merged into RoPE
 * (phase tables).  Only some of them NULL is ROTATTN_E_NULL.
 */
typedef struct rotattn_rope_rot {
  const float *cos_t, *sin_t, *cos_h, *sin_h, *cos_w, *sin_w;
  const float *rot_t, *rot_h, *rot_w;
} rotattn_rope_rot;

/*
 * Element strides of an fp16 [B][H][N][D] tensor whose channel stride is 1:
 * element (b, h, n, d) sits at b*batch + h*head + n*token + d.  A NULL
 * rotattn_strides* means contiguous [B][H][N][D] ({H*N*D, N*D, D}).  The
 * token-major output of a fused QKV projection, [B][N][3][H][D] with Q, K and
 * V starting at element 0, H*D and 2*H*D, is {N*3*H*D, D, 3*H*D}; an output
 * written as [B][N][H][D] for the output projection is {N*H*D, D, H*D}.
 * Every stride must be a multiple of 8 (16-byte rows, ROTATTN_E_ALIGN) and
 * token >= D (ROTATTN_E_ARG).  Outputs whose rows overlap are the caller's
 * error (not detected).
 */
typedef struct rotattn_strides {
  int64_t batch, head, token;
} rotattn_strides;

/*
 * Layout of the INT4 codes in a rotattn_prepared.
 *  ROTATTN_LAYOUT_PACKED: two codes per byte (4-bit two's complement); the
 *      attention kernel multiplies them on i8 MFMA.
 *  ROTATTN_LAYOUT_FP8: one code per byte, encoded as the FP8 E4M3 value of
 *      the integer (every integer in [-15, 15] is exact in E4M3); the attention
 *      kernel multiplies them on the f8f6f4 MFMA with fp32 accumulation.  The
 *      integer products and sums are the same exact integers as on i8 MFMA.
 *  ROTATTN_LAYOUT_FP6: the codes as FP6 E2M3 values (sign, 2 exponent bits
 *      with bias 1, 3 mantissa bits: every integer in [-7, 7] is exact); the
 *      kernel multiplies them on the f8f6f4 MFMA with both operands FP6, at
 *      twice the FP8 rate, with the same exact integer results.  Byte
 *      positions as in the FP8 layout, in groups of 32 codes: a group's 32
 *      bytes hold its 32 six-bit fields packed little-endian (field k in bits
 *      6k..6k+5 of bytes 0..23) and 8 zero bytes.
 */
typedef enum rotattn_layout {
  ROTATTN_LAYOUT_PACKED = 0,
  ROTATTN_LAYOUT_FP8 = 1,
  ROTATTN_LAYOUT_FP6 = 2
} rotattn_layout;

/*
 * Output of rotattn_prepare_qkv (device, caller-allocated; carve it from one
 * buffer with rotattn_prepared_carve).  NB = ceil(N/128), N_pad = 128*NB.
 *  layout: a rotattn_layout.
 *  q4, k4: INT4 codes in [-7, 7] of Q and K, rows N..N_pad-1 zero.
 *          PACKED: [B*H][N_pad][D/2] bytes.  Each group of 8 consecutive
 *          channels 8g..8g+7 occupies 4 bytes; byte i holds channel 8g+i in
 *          its low nibble and 8g+4+i in its high nibble.
 *          FP8: [B*H][N_pad][D] bytes, E4M3 of the code, channel order.
 *          FP6: [B*H][N_pad][D] bytes, group g of a row = channels
 *          32g..32g+31, channel 32g+k in field k.
 *  v4:     V codes per 128-token block, transposed (channel-major).
 *          PACKED: [B*H][NB][D][64]: row d holds the 128 keys of the block
 *          packed along keys as above (byte i of group g = keys 8g+i, 8g+4+i).
 *          FP8: [B*H][NB][D][128]: row d holds the block's 128 keys as E4M3
 *          codes, each 64-key half in the operand order of the P.V product
 *          (P as FP6): byte 32h+j (h in {0,1}, j < 32) is key
 *          32h + 8(j%16/4) + 4(j/16) + j%4.
 *          FP6: [B*H][NB][D][128]: row d in four groups g = 2c+h (c, h in
 *          {0,1}); field k of group g is key 64c + 32(k/16) + 8(k%16/4) +
 *          4h + k%4.
 *  rot64:  library scratch (its size is part of rotattn_prepared_bytes): the
 *          rotation and the RoPE tables rearranged for the prologue, refilled
 *          by every rotattn_prepare_qkv call that has a head to quantize.
 *  q_scale_l2, k_scale, v_scale: [B*H][NB] fp32 block scales (amax/7).
 *          q_scale_l2 = fl(q_scale * kappa), kappa = fl32(log2(e)/sqrt(D)), so
 *          that 2^(I * q_scale_l2 * k_scale) = exp(QK^T / sqrt(D)).
 *  q_rope, k_rope: [B*H][N_pad][D] fp16 RoPE'd (not rotated, not quantized)
 *          Q/K, rows N..N_pad-1 zero.
 *  v_t:    [B*H][N_pad/64][D][64] fp16: V transposed per 64-key tile, row d
 *          holding the tile's keys in the operand order of the fp16 P.V
 *          product: position 32s + 4c + i (s, i in {0..1}, {0..3}, c < 8) is
 *          key 32s + 4c' + i, c' = c with its two low bits swapped; keys >= N
 *          zero.
 *          q_rope, k_rope and v_t are written for fallback heads only and may
 *          be NULL when no head falls back.
 */
typedef struct rotattn_prepared {
  int32_t layout;
  uint8_t *q4, *k4, *v4;
  float *q_scale_l2, *k_scale, *v_scale;
  uint16_t *q_rope, *k_rope, *v_t;
  double *rot64;
} rotattn_prepared;

/*
 * Integer dumps of one (b, h, q_block) for parity checks (device,
 * caller-allocated); pass NULL in production.  Rows are the 128 queries of
 * the block (rows past N are written but meaningless).
 *  s_int:  [128][N_pad] int32 I = q-codes . k-codes (exact)
 *  p_code: [128][N_pad] uint8 P codes in [0, 15] (0 for keys >= N)
 *  pv_int: [NB][128][D] int32 per-key-tile sum_j code_ij * v-code_jd (exact)
 *  m_final, l_final: [128] fp32 final running max (log2 units) and normalizer
 */
typedef struct rotattn_debug {
  int32_t b, h, q_block;
  int32_t *s_int;
  uint8_t *p_code;
  int32_t *pv_int;
  float *m_final, *l_final;
} rotattn_debug;

/* Host-only shape check; needs no GPU.  Returns a rotattn_status. */
int rotattn_validate(const rotattn_shape* s);

/* Human-readable name of a status code (static string). */
const char* rotattn_strerror(int status);

/*
 * Host: fill RoPE tables (host arrays of the sizes in rotattn_rope_rot) with
 * the exact cos/sin of p * base^(-2j/d_a), rounded once to fp32 (computed in
 * long double).
 */
int rotattn_rope_tables_host(const rotattn_shape* s, double base,
                             float* cos_t, float* sin_t, float* cos_h,
                             float* sin_h, float* cos_w, float* sin_w);

/*
 * Host: RoPE tables with a rotation merged in (the RotateAttention page,
 * Abstract, offers rotation matrices that can be fused into RoPE).  A
 * block-diagonal rotation made of one 2x2 rotation by phi_{a,j} per RoPE pair
 * commutes with RoPE, so applying it after RoPE at position p equals RoPE with
 * angle p * theta_{a,j} + phi_{a,j}.  phase_a: host array of d_a/2 doubles
 * (NULL: all zero); entries are cos/sin of that angle computed in long double
 * and rounded once to fp32.  Use with rot_t = rot_h = rot_w = NULL.
 * Returns ROTATTN_E_ARG for a non-finite phase or base <= 1.
 */
int rotattn_rope_tables_phase_host(const rotattn_shape* s, double base,
                                   const double* phase_t, const double* phase_h,
                                   const double* phase_w, float* cos_t,
                                   float* sin_t, float* cos_h, float* sin_h,
                                   float* cos_w, float* sin_w);

/*
 * Host: the 15 P-code thresholds tau_k (smallest fp32 with 15*2^tau_k >=
 * k - 1/2), so code(x) = #{k : x >= tau_k} = rne(15 * 2^x) for x <= 0.
 */
int rotattn_pcode_thresholds_host(float tau[15]);

/* Host: kappa = fl32(log2(e)/sqrt(D)). */
float rotattn_kappa_host(int32_t D);

/* Bytes for the prepared buffers rotattn_prepare_qkv writes in the production
 * form: FP6 layout with the fp16 fallback buffers (q_rope, k_rope, v_t); 0 for
 * an invalid shape.  Equal to rotattn_workspace_bytes. */
size_t rotattn_prepared_bytes(const rotattn_shape* s);

/* Bytes for a rotattn_prepared of the given rotattn_layout (with_rope != 0
 * adds the fp16 fallback buffers); 0 for an invalid shape or layout. */
size_t rotattn_prepared_bytes_layout(const rotattn_shape* s, int with_rope, int layout);

/* Lay a rotattn_prepared out in [base, base+bytes) (256-byte aligned parts). */
int rotattn_prepared_carve(const rotattn_shape* s, void* base, size_t bytes,
                           int with_rope, int layout, rotattn_prepared* out);

/*
 * Prologue.  For every head with fallback_mask_host[b*H+h] == 0 (or all heads
 * when the mask is NULL): 3D RoPE on Q and K in fp32, the partition-wise
 * rotation (fp64 accumulation, one rounding to fp32; skipped when the
 * rotation pointers are NULL), per-block symmetric
 * INT4 quantization of Q, K, V, stored in out->layout.  For a fallback head:
 * RoPE'd fp16 Q'/K' into out->q_rope / out->k_rope and V^T tiles into
 * out->v_t only.
 */
int rotattn_prepare_qkv(const rotattn_shape* s, const uint16_t* q,
                        const uint16_t* k, const uint16_t* v,
                        const rotattn_rope_rot* rr,
                        const uint8_t* fallback_mask_host,
                        const rotattn_prepared* out, hipStream_t stream);

/* rotattn_prepare_qkv on q, k, v laid out with qkv_strides (shared by the
 * three; NULL = contiguous), e.g. read straight from a fused QKV projection's
 * token-major output with no transposition pass. */
int rotattn_prepare_qkv_strided(const rotattn_shape* s, const uint16_t* q,
                                const uint16_t* k, const uint16_t* v,
                                const rotattn_strides* qkv_strides,
                                const rotattn_rope_rot* rr,
                                const uint8_t* fallback_mask_host,
                                const rotattn_prepared* out,
                                hipStream_t stream);

/*
 * The DiT block's QKV projection with the prologue as its epilogue, in one
 * launch (RotateAttention page, Abstract: the INT4 attention inside the DiT
 * block, end to end): Q, K and V are never written to memory.  For every
 * 128-token block of every batch entry and every (Q|K|V, head), a work-group
 * computes the projection tile x . w^T (+ bias) on fp16 MFMA with fp32
 * accumulation, rounds it once to fp16 (round to nearest even) and runs the
 * prologue on it in LDS, writing `out` exactly as rotattn_prepare_qkv writes
 * it for those fp16 Q, K, V (codes and scales, or for fallback heads the
 * RoPE'd Q', K' and the V^T tiles).
 *  x:       fp16 [B][N][C] input, element strides x_batch and x_token (channel
 *           stride 1; multiples of 8; x_token <= 2^24), 16-byte aligned.
 *  C:       model width, a multiple of 64 (<= x_token).
 *  w:       fp16 [3*H*D][C], row r = output channel r: rows h*D + d are head
 *           h's Q channel d, then H*D rows of K, then H*D rows of V (a fused
 *           QKV linear layer's weight); 16-byte aligned.
 *  bias:    fp16 [3*H*D] in the same order, or NULL.
 *  qkv_out: NULL, or fp16 [3][B*H][N_pad][D] (16-byte aligned) that receives
 *           the rounded projection, rows >= N zero: Q, K and V per head as the
 *           prologue saw them.
 * Only D = 128 with the (44, 42, 42) split; other shapes return
 * ROTATTN_E_UNSUPPORTED.  Argument errors are returned before anything is
 * enqueued.
 */
int rotattn_qkv_proj_prepare(const rotattn_shape* s, const uint16_t* x,
                             int64_t x_batch, int64_t x_token, int32_t C,
                             const uint16_t* w, const uint16_t* bias,
                             const rotattn_rope_rot* rr,
                             const uint8_t* fallback_mask_host,
                             const rotattn_prepared* out, uint16_t* qkv_out,
                             hipStream_t stream);

/*
 * INT4 attention over the heads with fallback_mask_host[...] == 0 (all heads
 * when NULL): I = q4.k4^T (i8 MFMA for the PACKED layout, f8f6f4 MFMA for
 * FP8 and FP6), one-pass online softmax over 128-key tiles in the log2 domain, P codes
 * rne(15*2^(s-m)) against the running max, PV = codes.v4 on the same MFMA
 * kind, O = acc / l written as fp16 into o [B][H][N][D].
 * dbg != NULL additionally runs one instrumented work-group for (dbg->b,
 * dbg->h, dbg->q_block) that fills the integer dumps.
 */
int rotattn_int4_fwd(const rotattn_shape* s, const rotattn_prepared* p,
                     const uint8_t* fallback_mask_host, uint16_t* o,
                     const rotattn_debug* dbg, hipStream_t stream);

/*
 * Options of the INT4 attention.  normalizer: ROTATTN_NORM_EXP (default) takes
 * l as the sum of the unquantized 2^x; ROTATTN_NORM_CODES as the sum of the
 * P codes / 15, so that O is the quantized P's weighted mean of V (the other
 * reading of the quantized FlashAttention on the RotateAttention page,
 * Abstract; FP8 and FP6 layouts only, ROTATTN_E_UNSUPPORTED for PACKED).
 */
typedef enum rotattn_normalizer {
  ROTATTN_NORM_EXP = 0,
  ROTATTN_NORM_CODES = 1
} rotattn_normalizer;

typedef struct rotattn_int4_opts {
  int32_t normalizer;
} rotattn_int4_opts;

/* rotattn_int4_fwd writing o with o_strides (NULL = contiguous), e.g. as the
 * token-major [B][N][H][D] input of the output projection; opts NULL = the
 * defaults.  ROTATTN_E_ARG for an unknown normalizer. */
int rotattn_int4_fwd_strided(const rotattn_shape* s, const rotattn_prepared* p,
                             const uint8_t* fallback_mask_host, uint16_t* o,
                             const rotattn_strides* o_strides,
                             const rotattn_int4_opts* opts,
                             const rotattn_debug* dbg, hipStream_t stream);

/*
 * FP16 FlashAttention on the caller's tensors (RotateAttention page,
 * Abstract: selective FP16 fallback for accuracy-sensitive attention):
 * O = softmax(Q'K'^T / sqrt(D)) V on fp16 MFMA with fp32 softmax and
 * accumulation, for the heads with head_select_host[b*H+h] != 0 (all heads
 * when NULL).
 *  q_rope, k_rope: RoPE'd fp16 Q' and K' [B][H][N][D] (no rotation, no
 *          quantization -- what a fallback head of rotattn_prepare_qkv gets);
 *  v:      fp16 V [B][H][N][D];
 *  workspace: device scratch of at least rotattn_fp16_workspace_bytes(s)
 *          bytes, 16-byte aligned, caller-owned; the call stages zero-padded
 *          Q', K' and the V^T tiles of the P.V operand there (contents on
 *          return are unspecified);
 *  o:      fp16 [B][H][N][D], written for the selected heads only.
 * ROTATTN_E_WORKSPACE when the workspace is too small.
 */
int rotattn_fp16_fwd(const rotattn_shape* s, const uint16_t* q_rope, const uint16_t* k_rope,
                     const uint16_t* v, const uint8_t* head_select_host, void* workspace,
                     size_t workspace_bytes, uint16_t* o, hipStream_t stream);

/* rotattn_fp16_fwd with strides for q_rope, k_rope and v (shared; NULL =
 * contiguous) and for o (NULL = contiguous). */
int rotattn_fp16_fwd_strided(const rotattn_shape* s, const uint16_t* q_rope,
                             const uint16_t* k_rope, const uint16_t* v,
                             const rotattn_strides* qkv_strides, const uint8_t* head_select_host,
                             void* workspace, size_t workspace_bytes, uint16_t* o,
                             const rotattn_strides* o_strides, hipStream_t stream);

/* Workspace bytes for rotattn_fp16_fwd: three [B*H][N_pad][D] fp16 arrays
 * (256-byte aligned parts); 0 for an invalid shape. */
size_t rotattn_fp16_workspace_bytes(const rotattn_shape* s);

/*
 * rotattn_fp16_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same staging and FP16 attention (identical output), with the staging in
 * a static device array of ROTATTN_NOALLOC_SCRATCH_BYTES held by each GPU the
 * library runs on until the process ends, heads processed in chunks that fit
 * it, all on `stream`.  Q', K', V and O contiguous [B][H][N][D].  No
 * allocation and no synchronization; the scratch's device address is looked
 * up once per device.  ROTATTN_E_SCRATCH when one head's staging (three
 * [N_pad][D] fp16 arrays) exceeds the scratch (N_pad * D > 44,739,242 values).
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 */
int rotattn_fp16_fwd_noalloc(const rotattn_shape* s, const uint16_t* q_rope,
                             const uint16_t* k_rope, const uint16_t* v,
                             const uint8_t* head_select_host, uint16_t* o, hipStream_t stream);

/*
 * The same FP16 attention on prepared buffers: reads p->q_rope, p->k_rope
 * and p->v_t as written by rotattn_prepare_qkv for the selected heads
 * (fallback heads); no staging.  o: [B][H][N][D] fp16.
 */
int rotattn_fp16_fwd_prepared(const rotattn_shape* s, const rotattn_prepared* p,
                              const uint8_t* head_select_host, uint16_t* o,
                              hipStream_t stream);

/* rotattn_fp16_fwd_prepared writing o with o_strides (NULL = contiguous). */
int rotattn_fp16_fwd_prepared_strided(const rotattn_shape* s, const rotattn_prepared* p,
                                      const uint8_t* head_select_host, uint16_t* o,
                                      const rotattn_strides* o_strides, hipStream_t stream);

/* Workspace bytes for rotattn_mixed_fwd (an FP6-layout rotattn_prepared with
 * the fp16 fallback buffers). */
size_t rotattn_workspace_bytes(const rotattn_shape* s);

/*
 * Whole forward: prepare (FP6 layout), INT4 attention for mask == 0 heads,
 * FP16 attention for mask != 0 heads, all on `stream`, writing every head of o.
 * Every argument of the three steps is checked before the first launch.
 */
int rotattn_mixed_fwd(const rotattn_shape* s, const uint16_t* q,
                      const uint16_t* k, const uint16_t* v,
                      const rotattn_rope_rot* rr,
                      const uint8_t* fallback_mask_host, void* workspace,
                      size_t workspace_bytes, uint16_t* o, hipStream_t stream);

/* rotattn_mixed_fwd with input strides (shared by q, k, v) and output strides
 * (NULL = contiguous): one call between a fused QKV projection and the output
 * projection with no layout passes. */
int rotattn_mixed_fwd_strided(const rotattn_shape* s, const uint16_t* q,
                              const uint16_t* k, const uint16_t* v,
                              const rotattn_strides* qkv_strides,
                              const rotattn_rope_rot* rr,
                              const uint8_t* fallback_mask_host,
                              void* workspace, size_t workspace_bytes,
                              uint16_t* o, const rotattn_strides* o_strides,
                              hipStream_t stream);

/*
 * Self-test of the P-code device function (the exact code the attention
 * kernel of `layout` uses).  Evaluates code(x) for x = -magnitude over the
 * magnitude bit patterns [mag_lo, mag_lo + count) with c = 1, m = 0, and
 * records every position where the code changes: transitions[3*i] =
 * magnitude bits, [3*i+1] = code before, [3*i+2] = code after, for
 * i < max_transitions.  *n_transitions (device) receives the total count
 * (zero it first).
 */
int rotattn_pcode_sweep(int layout, uint32_t mag_lo, uint32_t count,
                        uint32_t* transitions, uint32_t max_transitions,
                        uint32_t* n_transitions, hipStream_t stream);

/*
 * Self-test: P codes of raw integer scores through the code path of the
 * attention kernel of `layout`.  I: [n] int32 exact QK^T values, c: fl(q_scale_l2*k_scale),
 * m: running max (log2 units, >= fl(I*c) for every element).  codes: [n]
 * uint8.  n must be a multiple of 4096.
 */
int rotattn_pcode_eval(int layout, const int32_t* I, uint32_t n, float c,
                       float m, uint8_t* codes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ROTATTN_H */

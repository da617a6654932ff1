"""CPU oracle for RotateAttention's mixed-precision INT4 FlashAttention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
The HIP path never calls it, and the two share no code: this file is plain
numpy (float64 unless a step fixes float32) plus mpmath for constants, written
from the pages, and it is deliberately slow and obvious.

Sources (page titles; every function cites the passage it follows):

[RA]  "RotateAttention: RoPE-Aware Rotation and Range Rectification for INT4
      Quantized Attention in Video Generation" -- Abstract.  It states the
      problem (attention in DiT video models with 3D RoPE), the RoPE-aware
      rotation of Q and K, the range-optimized quantization of the non-negative
      P = exp(QK - max(QK)) with a fixed scale and zero point, quantized
      FlashAttention, and selective FP16 fallback.
[WIN] mlsift.com RoPE page, first abstract (per-RoPE-wavelength distance
      window): with RoPE, a query-key score is exactly the sum of one term per
      2-D frequency pair.
[VC]  MXAttention page, VC-Attention abstract: V outliers are not tied to
      channels or positions; on large GPUs the float exponential between the
      two low-bit products is the slowest stage.

The pages give an abstract only: no equations, block sizes or kernel details.
Every step they leave open takes the plainest reading the rest supports; the
readings are these, repeated next to the code that takes them:

R1  S = Q K^T / sqrt(D); the max is the row max.  Work in the log2 domain:
    kappa = fl32(log2(e)/sqrt(D)) is folded into Q's scale, so
    exp(S - max S) == 2^(s - max s).
R2  3D RoPE: channels split into contiguous partitions [t | h | w]; inside a
    partition channels (2j, 2j+1) form a pair rotated by p_a * theta_{a,j},
    theta_{a,j} = 10000^(-2j/d_a); positions start at 0; token n is
    (t, h, w) with w fastest.
R3  Rotation after RoPE, inside each partition, same orthogonal matrix for Q
    and K (and every head); V is not rotated.
R4  Symmetric INT4: one fp32 scale per 128-token block x all channels per
    (batch, head) for each of Q, K, V; codes in [-7, 7].
R5  P code = rne(15 * 2^x) with x = s - m against the running max after the
    current key tile (one-pass online softmax), scale 1/15, zero point 0.
R6  Normalizer l = sum of the unquantized 2^x.
R7  FP16 fallback: plain softmax attention on RoPE'd fp16 Q/K (no rotation,
    no quantization), per (batch, head).
R8  The step before the attention in the DiT block (the pages place the
    attention inside it and quote end-to-end figures, nothing more): the
    usual fused linear layer, [Q | K | V] = x W^T + b with W's rows in the
    order Q heads, K heads, V heads and head h taking channels h*D..h*D+D-1
    of each; each output is the exact sum rounded once to fp16.

Exact rounding rules (so that codes are well defined bit for bit):
* RoPE in float32, no fused multiply-add:
  y0 = fl(fl(x0*c) - fl(x1*s)),  y1 = fl(fl(x0*s) + fl(x1*c)).
* Rotation: z = fl32(sum_k R[r,k] * y[k]), summed in float64 with k ascending
  (each product of two float32 values is exact in float64), one rounding to
  float32 at the end.
* Quantize: inv = fl(7/amax), scale = fl(amax/7) (correctly rounded), code =
  clamp(rne(fl(z*inv)), -7, 7); amax == 0 gives scale 0 and all-zero codes.
* Scores: c_t = fl(q_scale_l2 * k_scale_t), s = fl(fp32(I) * c_t),
  x = fl(s - m_new) in float32.
"""
from __future__ import annotations

import math

import mpmath
import numpy as np

L_BLOCK = 128           # quantization block length == key tile length (R4, R5)
ROPE_BASE = 10000.0     # R2
P_LEVELS = 15           # R5: unsigned INT4, scale 1/15, zero point 0

mpmath.mp.dps = 50


# --------------------------------------------------------------------------
# float32 rounding of exact (mpmath) values
# --------------------------------------------------------------------------

def _f32_neighbors(f: np.float32):
    up = np.nextafter(f, np.float32(np.inf), dtype=np.float32)
    dn = np.nextafter(f, np.float32(-np.inf), dtype=np.float32)
    return dn, up


def nearest_f32(v) -> np.float32:
    """The float32 nearest to the real number v (ties to even)."""
    v = mpmath.mpf(v)
    f = np.float32(float(v))
    best = None
    for c in (f, *_f32_neighbors(f)):
        d = abs(mpmath.mpf(float(c)) - v)
        key = (d, int(np.frombuffer(np.float32(c).tobytes(), np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def ceil_f32(v) -> np.float32:
    """The smallest float32 >= the real number v."""
    v = mpmath.mpf(v)
    f = np.float32(float(v))
    while mpmath.mpf(float(f)) < v:
        f = np.nextafter(f, np.float32(np.inf), dtype=np.float32)
    while True:
        dn = np.nextafter(f, np.float32(-np.inf), dtype=np.float32)
        if mpmath.mpf(float(dn)) >= v:
            f = dn
        else:
            return np.float32(f)


# --------------------------------------------------------------------------
# token grid and 3D RoPE  [RA: DiT video models with 3D RoPE; WIN: pairs]
# --------------------------------------------------------------------------

def partition_offsets(split):
    d_t, d_h, _ = split
    return (0, d_t, d_t + d_h)


def token_coords(grid):
    """(t, h, w) of every token, w fastest (R2)."""
    T, Hg, Wg = grid
    n = np.arange(T * Hg * Wg, dtype=np.int64)
    return n // (Hg * Wg), (n // Wg) % Hg, n % Wg


def rope_tables(extent: int, width: int, base: float = ROPE_BASE, dtype=np.float32,
                phase=None):
    """cos/sin of p * theta_j + phi_j for p < extent, j < width/2 (R2).

    theta_j = base^(-2j/width) taken as a real number; each entry is the exact
    cosine/sine rounded once to float32 (or float64 for the invariance pins).
    phase (float64 per pair, default 0) is a 2x2 rotation of each RoPE pair
    merged into RoPE (RotateAttention, Abstract: rotation matrices that can be
    fused into RoPE; see pair_rotation).
    """
    half = width // 2
    cos = np.empty((extent, half), dtype)
    sin = np.empty((extent, half), dtype)
    for j in range(half):
        theta = mpmath.power(mpmath.mpf(base), -mpmath.mpf(2 * j) / width)
        phi = mpmath.mpf(0) if phase is None else mpmath.mpf(float(phase[j]))
        for p in range(extent):
            ang = p * theta + phi
            if dtype == np.float32:
                cos[p, j] = nearest_f32(mpmath.cos(ang))
                sin[p, j] = nearest_f32(mpmath.sin(ang))
            else:
                cos[p, j] = float(mpmath.cos(ang))
                sin[p, j] = float(mpmath.sin(ang))
    return cos, sin


def all_rope_tables(grid, split, base: float = ROPE_BASE, dtype=np.float32, phases=None):
    """[(cos_t, sin_t), (cos_h, sin_h), (cos_w, sin_w)]; phases: one per-pair
    array per partition (a merged rotation) or None."""
    if phases is None:
        phases = [None, None, None]
    return [rope_tables(extent, width, base, dtype, ph)
            for extent, width, ph in zip(grid, split, phases)]


def pair_rotation(split, phases) -> list:
    """The rotation that phase tables merge into RoPE, as explicit matrices.

    One float64 [d_a, d_a] matrix per partition, block diagonal with the 2x2
    rotation [[cos phi_j, -sin phi_j], [sin phi_j, cos phi_j]] on pair
    (2j, 2j+1).  It commutes with RoPE at every position (both rotate the same
    planes), so applying it after RoPE equals RoPE with angle p*theta_j + phi_j
    (RotateAttention, Abstract: mergeable rotation fused into RoPE).
    """
    mats = []
    for width, ph in zip(split, phases):
        r = np.zeros((width, width))
        for j in range(width // 2):
            c, s = math.cos(float(ph[j])), math.sin(float(ph[j]))
            r[2 * j, 2 * j], r[2 * j, 2 * j + 1] = c, -s
            r[2 * j + 1, 2 * j], r[2 * j + 1, 2 * j + 1] = s, c
        mats.append(r)
    return mats


def apply_rope(x: np.ndarray, tables, grid, split) -> np.ndarray:
    """3D RoPE on [N, D] rows (R2), in the dtype of x and the tables.

    In float32 this is exactly y0 = fl(fl(x0*c) - fl(x1*s)),
    y1 = fl(fl(x0*s) + fl(x1*c)): numpy rounds every product and sum and
    never fuses them.
    """
    pos = token_coords(grid)
    y = np.empty_like(x)
    for a, (off, width) in enumerate(zip(partition_offsets(split), split)):
        cos_a, sin_a = tables[a]
        c = cos_a[pos[a]]
        s = sin_a[pos[a]]
        x0 = x[:, off:off + width:2]
        x1 = x[:, off + 1:off + width:2]
        y[:, off:off + width:2] = x0 * c - x1 * s
        y[:, off + 1:off + width:2] = x0 * s + x1 * c
    return y


# --------------------------------------------------------------------------
# RoPE-aware rotation  [RA: RoPE-aware Rotation -- cheap orthogonal matrices
# that spread the Q/K outliers RoPE's partitions concentrate, without
# disturbing RoPE]
# --------------------------------------------------------------------------

def rotate(y: np.ndarray, mats, split, out_dtype=np.float32) -> np.ndarray:
    """z = blockdiag(R_t, R_h, R_w) y per token (R3).

    Summed in float64 with k ascending; with float32 inputs every product is
    exact, and z is rounded once to out_dtype.  With float64 inputs and
    out_dtype float64 this is the plain float64 product used by the pins.
    """
    z = np.empty(y.shape, out_dtype)
    for off, width, r in zip(partition_offsets(split), split, mats):
        ya = y[:, off:off + width].astype(np.float64)
        ra = np.asarray(r, np.float64)
        acc = np.zeros((y.shape[0], width), np.float64)
        for k in range(width):
            acc = acc + ya[:, k:k + 1] * ra[:, k][None, :]
        z[:, off:off + width] = acc.astype(out_dtype)
    return z


# --------------------------------------------------------------------------
# symmetric INT4 quantization  [RA: low-bit quantization of Q, K; R4]
# --------------------------------------------------------------------------

def quantize_blocks(z: np.ndarray, block: int = L_BLOCK):
    """Per-block symmetric INT4 of [N, D] float32 rows.

    Returns (codes int8 [N, D], scale float32 [nb], inv float32 [nb]).  The
    last block may be partial; its amax is over the valid rows only.
    """
    z = np.asarray(z, np.float32)
    N = z.shape[0]
    nb = -(-N // block)
    codes = np.zeros(z.shape, np.int8)
    scale = np.zeros(nb, np.float32)
    inv = np.zeros(nb, np.float32)
    for b in range(nb):
        blk = z[b * block:min(N, (b + 1) * block)]
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        if amax == 0:
            continue
        inv[b] = np.float32(7) / amax
        scale[b] = amax / np.float32(7)
        codes[b * block:b * block + blk.shape[0]] = np.clip(np.rint(blk * inv[b]), -7, 7).astype(np.int8)
    return codes, scale, inv


def kappa(D: int) -> np.float32:
    """fl32(log2(e) / sqrt(D)) (R1)."""
    return nearest_f32(mpmath.log(mpmath.e, 2) / mpmath.sqrt(D))


# --------------------------------------------------------------------------
# range-optimized P quantization  [RA: Range-optimized P Quantization -- P is
# never negative, so a symmetric code would leave half of the 4-bit levels
# unused; a fixed scale and zero point use all 16]
# --------------------------------------------------------------------------

_THRESHOLDS = None


def pcode_thresholds() -> np.ndarray:
    """tau_k, k = 1..15: the smallest float32 with 15 * 2^tau_k >= k - 1/2.

    code(x) = rne(15 * 2^x) = #{k : x >= tau_k} for x <= 0 (R5).  The only
    exact tie is k = 8 at x = -1 (7.5 rounds to the even 8).
    """
    global _THRESHOLDS
    if _THRESHOLDS is None:
        tau = [ceil_f32(mpmath.log(mpmath.mpf(2 * k - 1) / 30, 2)) for k in range(1, P_LEVELS + 1)]
        _THRESHOLDS = np.array(tau, np.float32)
    return _THRESHOLDS.copy()


def pcode(x: np.ndarray) -> np.ndarray:
    """uint8 P code of float32 x <= 0: clamp(rne(15 * 2^x), 0, 15) exactly."""
    tau = pcode_thresholds()
    return np.searchsorted(tau, np.asarray(x, np.float32), side="right").astype(np.uint8)


# --------------------------------------------------------------------------
# quantized FlashAttention, one-pass online softmax  [RA: quantized
# FlashAttention; P = exp(QK - max(QK)); R1, R5, R6]
# --------------------------------------------------------------------------

def int4_attention(q_codes, q_scale_l2, k_codes, k_scale, v_codes, v_scale, rows, *,
                   tile: int = L_BLOCK, quantize_p: bool = True, score_dtype=np.float32,
                   record: dict | None = None, int64_check: bool = False,
                   normalizer: str = "exp"):
    """Output rows of one (batch, head), key tiles in ascending order.

    q_codes/k_codes/v_codes: [N, D] integer codes (or any float values for the
    identity-quantizer pin), *_scale: per 128-token block.  rows: query rows.
    For each key tile t, with m = -inf, l = 0, acc = 0 at the start:
      I      = q_codes[rows] . k_codes[tile]^T            (exact integers)
      c      = fl(q_scale_l2[block(row)] * k_scale[t])
      s      = fl(I * c),  m_new = max(m, max_j s),  x = fl(s - m_new)
      alpha  = 2^(m - m_new)                              (0 on the first tile)
      l      = alpha * l + sum_j 2^x
      P      = code(x) / 15  (or 2^x when quantize_p is False)
      acc    = alpha * acc + v_scale[t] * P . v_codes[tile]
      m      = m_new
    then O = fp16(acc / l).  Keys past N never enter (partial last tile).
    The float part (alpha, l, acc) is evaluated in float64.

    normalizer "codes" takes l = alpha * l + sum_j code_j / 15 instead (R6's
    alternative: the normalizer of the quantized P, so that O is the
    code-weighted mean of the dequantized V rows).
    """
    if normalizer not in ("exp", "codes") or (normalizer == "codes" and not quantize_p):
        raise ValueError(normalizer)
    q_codes = np.asarray(q_codes)
    N, D = k_codes.shape
    rows = np.asarray(rows, np.int64)
    R = rows.size
    qb = rows // L_BLOCK
    m = np.full(R, -np.inf, score_dtype)
    l = np.zeros(R, np.float64)
    acc = np.zeros((R, D), np.float64)
    qi = q_codes[rows].astype(np.float64)
    qs = np.asarray(q_scale_l2, score_dtype)[qb]
    n_tiles = -(-N // tile)
    if record is not None:
        record.update(I=[], x=[], code=[], pv=[], m=[], l=[])
    for t in range(n_tiles):
        k0, k1 = t * tile, min(N, (t + 1) * tile)
        kt = k_codes[k0:k1].astype(np.float64)
        I = qi @ kt.T
        if quantize_p:
            assert np.all(I == np.rint(I)) and np.all(np.abs(I) < 2 ** 53)
            if int64_check:
                Ii = q_codes[rows].astype(np.int64) @ k_codes[k0:k1].astype(np.int64).T
                assert np.array_equal(Ii, I.astype(np.int64))
        ks = np.asarray(k_scale, score_dtype)[k0 // L_BLOCK] if tile == L_BLOCK else None
        if ks is None:
            # tile sizes other than the 128-token block: per-key scale lookup
            ks_keys = np.asarray(k_scale, score_dtype)[np.arange(k0, k1) // L_BLOCK]
            c = (qs[:, None] * ks_keys[None, :]).astype(score_dtype)
            s = (I.astype(score_dtype) * c).astype(score_dtype)
        else:
            c = (qs * ks).astype(score_dtype)
            s = (I.astype(score_dtype) * c[:, None]).astype(score_dtype)
        m_new = np.maximum(m, s.max(axis=1))
        x = (s - m_new[:, None]).astype(score_dtype)
        p = np.exp2(x.astype(np.float64))
        alpha = np.where(np.isneginf(m), 0.0, np.exp2(m.astype(np.float64) - m_new.astype(np.float64)))
        vt = v_codes[k0:k1].astype(np.float64)
        if quantize_p:
            code = pcode(x)
        if normalizer == "codes":
            l = alpha * l + code.astype(np.float64).sum(axis=1) / P_LEVELS
        else:
            l = alpha * l + p.sum(axis=1)
        if quantize_p:
            pv = code.astype(np.float64) @ vt
            assert np.all(pv == np.rint(pv))
            vs = np.float64(np.asarray(v_scale, np.float32)[k0 // L_BLOCK])
            acc = alpha[:, None] * acc + (vs / P_LEVELS) * pv
        else:
            code = None
            vs_keys = np.asarray(v_scale, np.float64)[np.arange(k0, k1) // L_BLOCK]
            pv = p @ (vt * vs_keys[:, None])
            acc = alpha[:, None] * acc + pv
        m = m_new
        if record is not None:
            record["I"].append(I.astype(np.int64) if quantize_p else I)
            record["x"].append(x)
            record["code"].append(code)
            record["pv"].append(pv.astype(np.int64) if quantize_p else pv)
            record["m"].append(m.copy())
            record["l"].append(l.copy())
    out = acc / l[:, None]
    if record is not None:
        record["acc"] = acc
        record["l_final"] = l
        record["m_final"] = m
    return out.astype(np.float16), out


def softmax_attention(q, k, v, rows, scale):
    """Plain two-pass softmax attention in float64: softmax(scale*QK^T) V."""
    qr = np.asarray(q, np.float64)[np.asarray(rows, np.int64)]
    S = (qr @ np.asarray(k, np.float64).T) * scale
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P @ np.asarray(v, np.float64)) / P.sum(axis=1, keepdims=True)


def fp16_attention(q_rope16, k_rope16, v16, rows):
    """FP16 fallback head (R7): softmax(Q'K'^T/sqrt(D)) V exactly, rounded to fp16."""
    D = q_rope16.shape[1]
    out = softmax_attention(q_rope16, k_rope16, v16, rows, 1.0 / math.sqrt(D))
    return out.astype(np.float16), out


# --------------------------------------------------------------------------
# the QKV projection before the attention  [R8]
# --------------------------------------------------------------------------

def qkv_projection(x16, w16, b16=None):
    """R8: x [n, C] fp16, W [3 H D, C] fp16 (row r = output channel r), b
    [3 H D] fp16 or None -> fp16 [n, 3 H D]: the float64 sum over C (+ b),
    rounded once to fp16 (round to nearest even).  Every product of two fp16
    values is exact in float64; the sum is exact too whenever it needs no more
    than float64's 53 bits (the tests' exact cases), else within float64's
    own error, far below fp16's rounding."""
    acc = np.asarray(x16, np.float64) @ np.asarray(w16, np.float64).T
    if b16 is not None:
        acc = acc + np.asarray(b16, np.float64)[None, :]
    return acc.astype(np.float16)


def split_qkv(y16, H: int, D: int):
    """R8: the projection output [n, 3 H D] -> Q, K, V, each [H, n, D]."""
    n = y16.shape[0]
    t = np.asarray(y16).reshape(n, 3, H, D)
    return tuple(np.ascontiguousarray(t[:, i].transpose(1, 0, 2)) for i in range(3))


# --------------------------------------------------------------------------
# one head, end to end
# --------------------------------------------------------------------------

def prepare_head(q16, k16, v16, tables, mats32, grid, split, fallback: bool = False):
    """Prologue of one head: RoPE, rotation, INT4 quantization (R2-R4).

    mats32 None: no dense rotation, z = the RoPE'd values (the form of a
    rotation merged into the RoPE tables).  A fallback head only gets RoPE'd
    fp16 Q'/K' (R7).
    """
    D = q16.shape[1]
    yq = apply_rope(q16.astype(np.float32), tables, grid, split)
    yk = apply_rope(k16.astype(np.float32), tables, grid, split)
    if fallback:
        return {"q_rope": yq.astype(np.float16), "k_rope": yk.astype(np.float16)}
    zq = yq if mats32 is None else rotate(yq, mats32, split)
    zk = yk if mats32 is None else rotate(yk, mats32, split)
    qc, qs, _ = quantize_blocks(zq)
    kc, ks, _ = quantize_blocks(zk)
    vc, vs, _ = quantize_blocks(v16.astype(np.float32))
    return {"q_codes": qc, "k_codes": kc, "v_codes": vc,
            "q_scale_l2": (qs * kappa(D)).astype(np.float32),
            "k_scale": ks, "v_scale": vs, "zq": zq, "zk": zk}


def forward_head(q16, k16, v16, tables, mats32, grid, split, rows, fallback: bool = False,
                 record: dict | None = None):
    """O rows (fp16) of one head: INT4 RotateAttention, or the FP16 fallback."""
    prep = prepare_head(q16, k16, v16, tables, mats32, grid, split, fallback)
    if fallback:
        o16, _ = fp16_attention(prep["q_rope"], prep["k_rope"], v16, rows)
    else:
        o16, _ = int4_attention(prep["q_codes"], prep["q_scale_l2"], prep["k_codes"],
                                prep["k_scale"], prep["v_codes"], prep["v_scale"], rows,
                                record=record)
    return o16, prep

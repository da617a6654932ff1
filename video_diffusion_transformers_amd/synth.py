"""Seeded synthetic inputs for the RotateAttention INT4 attention forward.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no RoPE, no rotation, no quantization, no softmax), so both
the HIP path's tests and the CPU oracle's tests can take their inputs from it
without sharing any of the method's code.

Workload shapes follow the RotateAttention page (DiT video generation models
with 3D RoPE, Abstract) at Wan-class latent grids: 480p = 21x30x52 tokens and
720p = 21x45x80 tokens, 40 heads of width 128.  No trained weights or real
activations exist here, so Q/K/V are drawn from distributions that carry the
structure the pages describe:

* Q/K outliers sit in a few channels whose placement follows how 3D RoPE
  partitions the head dimension (RotateAttention page, Abstract) -- here four
  heavy channels inside the temporal partition, the same in Q and K, with the
  logit spread held at LOGIT_STD nats so that each query row spreads its
  weight over hundreds to thousands of the 75,600 keys at 720p instead of
  collapsing onto one;
* V outliers are not tied to channels or positions (MXAttention page,
  VC-Attention abstract) -- here sparse whole-token rows scaled up.

The "video_literal" distribution is the same recipe without the logit
calibration, with Q's and K's outlier channels drawn independently: rows are
then close to one-hot (logit spreads of tens of nats).

Every tensor of every head has its own stream,
``SeedSequence([cfg_seed, step, tensor, b, h])`` with tensor Q=0, K=1, V=2, so a
single head can be regenerated without the others; a head's Q/K channel scales
come from ``SeedSequence([cfg_seed, STRUCTURE_SALT, b, h])``.  Values are drawn in
float64, rounded to float32 and then to float16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Tuple

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
ROTATION_SEED = 7          # SeedSequence([7, partition]) for the default rotation
ROW_SAMPLE_SALT = 555      # SeedSequence([cfg_seed, 555, h]) for sampled query rows
MASK_SALT = 999            # SeedSequence([cfg_seed, 999]) for the fallback mask
PHASE_SALT = 444           # SeedSequence([seed, 444, partition]) for merged-rotation phases
STRUCTURE_SALT = 333       # SeedSequence([cfg_seed, 333, b, h]) for a head's Q/K channel scales
LOGIT_STD = 2.5            # nats: spread of q.k/sqrt(D) over independent rows ("video")


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: shape, value distribution and head routing."""
    name: str
    B: int
    H: int
    grid: Tuple[int, int, int]        # (T, Hg, Wg) latent token grid
    D: int
    split: Tuple[int, int, int]       # RoPE partition widths (d_t, d_h, d_w)
    dist: str                         # "tiny" | "video" | "video_literal" | "diffuse"
    cfg_seed: int
    sample_rows: int | None = None    # None: every query row is checked
    fallback: str = "none"            # "none" | "head1" | "quarter"
    steps: int = 1

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def BH(self) -> int:
        return self.B * self.H


CONFIGS = {
    # D=64 split 24/20/20, N(0,1) with 2 outlier channels per partition x20,
    # head 1 routed to the FP16 fallback.
    "tiny": Config("tiny", 1, 2, (2, 4, 4), 64, (24, 20, 20), "tiny", 0,
                   fallback="head1"),
    "small": Config("small", 1, 8, (4, 16, 16), 128, (44, 42, 42), "video", 1),
    "480p": Config("480p", 1, 40, (21, 30, 52), 128, (44, 42, 42), "video", 2,
                   sample_rows=512),
    "720p": Config("720p", 1, 40, (21, 45, 80), 128, (44, 42, 42), "video", 3,
                   sample_rows=256),
    "mixed": Config("mixed", 1, 40, (21, 45, 80), 128, (44, 42, 42), "video", 4,
                    sample_rows=256, fallback="quarter", steps=4),
    # the Small and 480p shapes on the recipe exactly as stated, without the
    # logit calibration of "video": per-channel lognormal scales and four
    # temporal outlier channels drawn afresh for every tensor (Q and K
    # independently), V as in "video"
    "small_lit": Config("small_lit", 1, 8, (4, 16, 16), 128, (44, 42, 42), "video_literal", 1),
    "480p_lit": Config("480p_lit", 1, 40, (21, 30, 52), 128, (44, 42, 42), "video_literal", 2,
                       sample_rows=512),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def _to_f16(x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float32).astype(np.float16)


def partition_offsets(split) -> Tuple[int, int, int]:
    d_t, d_h, _ = split
    return (0, d_t, d_t + d_h)


def _qk_tiny(rng, N, D, split):
    x = rng.standard_normal((N, D))
    for off, width in zip(partition_offsets(split), split):
        ch = rng.choice(width, size=2, replace=False) + off
        x[:, ch] *= 20.0
    return x


def _video_channel_scales(cfg: Config, b: int, h: int):
    """Per-channel standard deviations of one head's Q and K.

    They stand for the head's projection weights, so they come from a stream
    of their own, SeedSequence([cfg_seed, STRUCTURE_SALT, b, h]), and stay the
    same across denoising steps.  Each channel has a log-normal scale
    exp(0.5 z); four channels inside the temporal RoPE partition, the same four
    in Q and K, are raised by independent factors in [10, 30].  Q and K are then
    scaled by one common factor so that the scaled logits q.k/sqrt(D) of
    independent rows have a standard deviation of LOGIT_STD nats:
    Var(q.k/sqrt(D)) = sum_c sq_c^2 sk_c^2 / D for independent zero-mean rows.
    """
    D, split = cfg.D, cfg.split
    rng = _rng(cfg.cfg_seed, STRUCTURE_SALT, b, h)
    sq = np.exp(0.5 * rng.standard_normal(D))
    sk = np.exp(0.5 * rng.standard_normal(D))
    ch = rng.choice(split[0], size=4, replace=False)      # temporal partition
    sq[ch] *= rng.uniform(10.0, 30.0, size=4)
    sk[ch] *= rng.uniform(10.0, 30.0, size=4)
    logit_sd = np.sqrt(np.sum(sq ** 2 * sk ** 2) / D)
    c = np.sqrt(LOGIT_STD / logit_sd)
    return sq * c, sk * c


def _qk_video_literal(rng, N, D, split):
    """Q or K of the literal recipe, from the tensor's own stream: per-channel
    scale exp(0.5 z), four channels of the temporal partition (chosen without
    replacement) raised by independent factors in [10, 30], then
    x = scale * N(0, 1).  No rescaling of the logit spread."""
    sig = np.exp(0.5 * rng.standard_normal(D))
    ch = rng.choice(split[0], size=4, replace=False)
    sig[ch] *= rng.uniform(10.0, 30.0, size=4)
    return rng.standard_normal((N, D)) * sig[None, :]


def _v_video(rng, N, D):
    x = rng.standard_normal((N, D))
    n_out = max(1, int(round(0.002 * N)))
    rows = rng.choice(N, size=n_out, replace=False)
    x[rows, :] *= 15.0
    return x


def head_qkv(cfg: Config, step: int, b: int, h: int):
    """float16 Q, K, V of one (batch, head), each [N, D] row-major."""
    N, D = cfg.N, cfg.D
    out = []
    for tensor in (TENSOR_Q, TENSOR_K, TENSOR_V):
        rng = _rng(cfg.cfg_seed, step, tensor, b, h)
        if cfg.dist == "tiny":
            x = _qk_tiny(rng, N, D, cfg.split) if tensor != TENSOR_V else rng.standard_normal((N, D))
        elif cfg.dist == "video":
            if tensor == TENSOR_V:
                x = _v_video(rng, N, D)
            else:
                scales = _video_channel_scales(cfg, b, h)[0 if tensor == TENSOR_Q else 1]
                x = rng.standard_normal((N, D)) * scales[None, :]
        elif cfg.dist == "video_literal":
            x = _v_video(rng, N, D) if tensor == TENSOR_V else _qk_video_literal(rng, N, D, cfg.split)
        elif cfg.dist == "diffuse":
            # no outliers; scaled logits have a standard deviation of about
            # one nat, so rows are spread and every P code occurs
            x = rng.standard_normal((N, D))
        else:
            raise ValueError(cfg.dist)
        out.append(_to_f16(x))
    return tuple(out)


def all_heads_qkv(cfg: Config, step: int = 0, workers: int | None = None):
    """float16 Q, K, V for every head, each [B, H, N, D] contiguous.  Heads are
    drawn on a thread pool (each head has its own streams, so the result does
    not depend on the number of workers; numpy's generators release the GIL)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    shape = (cfg.B, cfg.H, cfg.N, cfg.D)
    q = np.empty(shape, np.float16)
    k = np.empty(shape, np.float16)
    v = np.empty(shape, np.float16)

    def one(bh):
        b, h = divmod(bh, cfg.H)
        q[b, h], k[b, h], v[b, h] = head_qkv(cfg, step, b, h)

    n = workers if workers is not None else min(16, len(os.sched_getaffinity(0)))
    if n <= 1 or cfg.BH == 1:
        for bh in range(cfg.BH):
            one(bh)
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(one, range(cfg.BH)))
    return q, k, v


def rotation_matrices(split, seed: int = ROTATION_SEED):
    """Seeded Haar-random orthogonal matrix per RoPE partition.

    Returned twice: float64 (for invariance checks) and float32 (what the
    pipeline consumes, the float64 matrix rounded once).  The same matrices are
    used for Q and K and for every head.  Haar sampling: QR of a Gaussian
    matrix with the signs of R's diagonal folded into Q.
    """
    r64, r32 = [], []
    for a, width in enumerate(split):
        g = _rng(seed, a).standard_normal((width, width))
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]
        r64.append(np.ascontiguousarray(qm))
        r32.append(np.ascontiguousarray(qm.astype(np.float32)))
    return r64, r32


def mergeable_phases(split, seed: int = ROTATION_SEED):
    """Seeded per-pair angles, uniform in [0, 2 pi), one float64 array of d_a/2
    per RoPE partition: the default rotation to merge into the RoPE tables.
    Stream: SeedSequence([seed, PHASE_SALT, partition])."""
    return [_rng(seed, PHASE_SALT, a).uniform(0.0, 2.0 * np.pi, size=width // 2)
            for a, width in enumerate(split)]


def fallback_mask(cfg: Config) -> np.ndarray:
    """uint8 [B*H]; nonzero routes that head to the FP16 fallback."""
    mask = np.zeros(cfg.BH, np.uint8)
    if cfg.fallback == "head1":
        mask[1::cfg.H] = 1
    elif cfg.fallback == "quarter":
        rng = _rng(cfg.cfg_seed, MASK_SALT)
        mask[rng.choice(cfg.BH, size=cfg.BH // 4, replace=False)] = 1
    elif cfg.fallback != "none":
        raise ValueError(cfg.fallback)
    return mask


def fallback_schedule(cfg: Config, n_steps: int, n_layers: int = 1, early_fp16_steps: int = 1,
                      fp16_layers=()) -> np.ndarray:
    """uint8 [n_steps, n_layers, B*H]: the fallback mask of every (denoising
    step, attention layer).  Full-precision fallback may be given to whole
    attention blocks and to whole denoising steps (RotateAttention page,
    Abstract); the plainest schedule of that kind is used here: the first
    early_fp16_steps steps and the layers listed in fp16_layers run every head
    in FP16, every other (step, layer) uses the config's fixed head mask."""
    if n_steps < 0 or n_layers < 1:
        raise ValueError("n_steps must be >= 0 and n_layers >= 1")
    sched = np.repeat(fallback_mask(cfg)[None, None, :], n_steps, axis=0)
    sched = np.repeat(sched, n_layers, axis=1)
    sched[:min(early_fp16_steps, n_steps)] = 1
    for layer in fp16_layers:
        if not 0 <= layer < n_layers:
            raise ValueError(f"layer {layer} out of range")
        sched[:, layer] = 1
    return sched


def sampled_rows(cfg: Config, h: int, count: int | None = None) -> np.ndarray:
    """Sorted query rows checked against the oracle for head h."""
    count = cfg.sample_rows if count is None else count
    if count is None or count >= cfg.N:
        return np.arange(cfg.N, dtype=np.int64)
    rng = _rng(cfg.cfg_seed, ROW_SAMPLE_SALT, h)
    return np.sort(rng.choice(cfg.N, size=count, replace=False)).astype(np.int64)


def projection_inputs(cfg: Config, C: int, kind: str = "normal", seed: int = 0):
    """Seeded inputs of the QKV projection before the attention: x fp16
    [B][N][C], w fp16 [3 H D][C] (Q heads, then K, then V), bias fp16 [3 H D].

    "normal": x ~ N(0, 1), w ~ N(0, 1/C), bias ~ N(0, 0.05^2) (a random-weight
    DiT layer: Q, K, V of unit scale).  "dyadic": x = a/64 and w = c/256,
    bias = e/256 with small integers a, c, e, so that every partial sum of
    a width up to 1024 is exact in float32 and the projection has one exact
    value whatever the summation order."""
    rng = _rng(cfg.cfg_seed, 7001, seed, C)
    R = 3 * cfg.H * cfg.D
    if kind == "normal":
        x = _to_f16(rng.standard_normal((cfg.B, cfg.N, C)))
        w = _to_f16(rng.standard_normal((R, C)) / np.sqrt(C))
        b = _to_f16(0.05 * rng.standard_normal(R))
    elif kind == "dyadic":
        if C > 1024:
            raise ValueError("dyadic projection inputs are exact up to C = 1024")
        x = (rng.integers(-32, 33, (cfg.B, cfg.N, C)) / 64.0).astype(np.float16)
        w = (rng.integers(-8, 9, (R, C)) / 256.0).astype(np.float16)
        b = (rng.integers(-64, 65, R) / 256.0).astype(np.float16)
    else:
        raise ValueError(kind)
    return x, w, b


def custom_config(name, B, H, grid, D, split, dist="video", cfg_seed=11, **kw) -> Config:
    """A config outside the named set (ragged tails, fuzzing)."""
    return Config(name, B, H, tuple(grid), D, tuple(split), dist, cfg_seed, **kw)

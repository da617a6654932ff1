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
  partitions the head dimension (RotateAttention page, Abstract) -- here a
  few heavy channels inside one partition;
* V outliers are not tied to channels or positions (MXAttention page,
  VC-Attention abstract) -- here sparse whole-token rows scaled up.

Every tensor of every head has its own stream,
``SeedSequence([cfg_seed, step, tensor, b, h])`` with tensor Q=0, K=1, V=2, so a
single head can be regenerated without the others.  Values are drawn in
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


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: shape, value distribution and head routing."""
    name: str
    B: int
    H: int
    grid: Tuple[int, int, int]        # (T, Hg, Wg) latent token grid
    D: int
    split: Tuple[int, int, int]       # RoPE partition widths (d_t, d_h, d_w)
    dist: str                         # "tiny" | "video" | "diffuse"
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


def _qk_video(rng, N, D, split):
    z = rng.standard_normal(D)
    x = rng.standard_normal((N, D)) * np.exp(0.5 * z)[None, :]
    ch = rng.choice(split[0], size=4, replace=False)      # temporal partition
    mult = rng.uniform(10.0, 30.0, size=4)
    x[:, ch] *= mult[None, :]
    return x


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
            x = _qk_video(rng, N, D, cfg.split) if tensor != TENSOR_V else _v_video(rng, N, D)
        elif cfg.dist == "diffuse":
            # no outliers; scaled logits have a standard deviation of about
            # one nat, so rows are spread and every P code occurs
            x = rng.standard_normal((N, D))
        else:
            raise ValueError(cfg.dist)
        out.append(_to_f16(x))
    return tuple(out)


def all_heads_qkv(cfg: Config, step: int = 0):
    """float16 Q, K, V for every head, each [B, H, N, D] contiguous."""
    shape = (cfg.B, cfg.H, cfg.N, cfg.D)
    q = np.empty(shape, np.float16)
    k = np.empty(shape, np.float16)
    v = np.empty(shape, np.float16)
    for b in range(cfg.B):
        for h in range(cfg.H):
            q[b, h], k[b, h], v[b, h] = head_qkv(cfg, step, b, h)
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


def sampled_rows(cfg: Config, h: int, count: int | None = None) -> np.ndarray:
    """Sorted query rows checked against the oracle for head h."""
    count = cfg.sample_rows if count is None else count
    if count is None or count >= cfg.N:
        return np.arange(cfg.N, dtype=np.int64)
    rng = _rng(cfg.cfg_seed, ROW_SAMPLE_SALT, h)
    return np.sort(rng.choice(cfg.N, size=count, replace=False)).astype(np.int64)


def custom_config(name, B, H, grid, D, split, dist="video", cfg_seed=11, **kw) -> Config:
    """A config outside the named set (ragged tails, fuzzing)."""
    return Config(name, B, H, tuple(grid), D, tuple(split), dist, cfg_seed, **kw)

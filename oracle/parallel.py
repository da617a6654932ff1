"""Process pool over the CPU oracle: reference output rows of many heads.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  Each worker regenerates its head's fp16 Q/K/V from the seeded generator
(``synth``, which holds none of the method's arithmetic) and runs the plain
oracle of ``rotattn_oracle`` on it -- the prologue of the head (3D RoPE, the
partition-wise rotation, per-block INT4 quantization) and then the INT4
attention, or the FP16 fallback attention, on the requested query rows.
Heads are independent, so the pool only distributes whole heads; it adds no
arithmetic of its own.  Workers are started with the "spawn" method (the
parent may hold a GPU context, which a forked child must not inherit) and
use one BLAS thread each.
"""
from __future__ import annotations

import functools
import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from . import rotattn_oracle as O

MAX_WORKERS = 16   # one GPU's share of a box's host cores


def host_cores() -> int:
    """Cores this process may run on."""
    return len(os.sched_getaffinity(0))


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


@functools.lru_cache(maxsize=8)
def _tables(grid, split, phases_key):
    phases = None if phases_key is None else [np.array(p) for p in phases_key]
    return O.all_rope_tables(grid, split, phases=phases)


@functools.lru_cache(maxsize=4)
def _rotation(split):
    from video_diffusion_transformers_amd import synth
    return synth.rotation_matrices(split)[1]


def head_job(cfg, step: int, bh: int, rows, fallback: bool, normalizer: str = "exp",
             merged: bool = False):
    """Reference rows of one head: (bh, fp16 rows [len(rows), D], seconds spent
    in the prologue, seconds spent in attention)."""
    from video_diffusion_transformers_amd import synth
    b, h = divmod(bh, cfg.H)
    q, k, v = synth.head_qkv(cfg, step, b, h)
    phases = synth.mergeable_phases(cfg.split) if merged else None
    key = None if phases is None else tuple(tuple(float(x) for x in p) for p in phases)
    tabs = _tables(tuple(cfg.grid), tuple(cfg.split), key)
    r32 = None if merged else _rotation(tuple(cfg.split))
    rows = np.asarray(rows, np.int64)
    t0 = time.perf_counter()
    prep = O.prepare_head(q, k, v, tabs, r32, cfg.grid, cfg.split, fallback=fallback)
    t1 = time.perf_counter()
    if fallback:
        o16, _ = O.fp16_attention(prep["q_rope"], prep["k_rope"], v, rows)
    else:
        o16, _ = O.int4_attention(prep["q_codes"], prep["q_scale_l2"], prep["k_codes"],
                                  prep["k_scale"], prep["v_codes"], prep["v_scale"], rows,
                                  normalizer=normalizer)
    t2 = time.perf_counter()
    return bh, o16, t1 - t0, t2 - t1


def run_heads(cfg, step: int, jobs, workers: int | None = None, normalizer: str = "exp",
              merged: bool = False):
    """jobs: iterable of (bh, rows, fallback).  Returns {bh: fp16 rows} and the
    per-head (prologue seconds, attention seconds)."""
    jobs = list(jobs)
    n = max(1, min(workers or host_cores(), MAX_WORKERS, len(jobs)))
    out, secs = {}, {}
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                             initializer=_init_worker) as ex:
        futs = [ex.submit(head_job, cfg, step, bh, rows, fb, normalizer, merged)
                for bh, rows, fb in jobs]
        for f in futs:
            bh, o16, tp, ta = f.result()
            out[bh] = o16
            secs[bh] = (tp, ta)
    return out, secs


def prep_job(cfg, step: int, bh: int, fallback: bool, merged: bool = False):
    """The oracle prologue of one head: codes and block scales (INT4 heads) or
    the RoPE'd fp16 Q'/K' (fallback heads); the unquantized z is dropped."""
    from video_diffusion_transformers_amd import synth
    b, h = divmod(bh, cfg.H)
    q, k, v = synth.head_qkv(cfg, step, b, h)
    phases = synth.mergeable_phases(cfg.split) if merged else None
    key = None if phases is None else tuple(tuple(float(x) for x in p) for p in phases)
    tabs = _tables(tuple(cfg.grid), tuple(cfg.split), key)
    r32 = None if merged else _rotation(tuple(cfg.split))
    prep = O.prepare_head(q, k, v, tabs, r32, cfg.grid, cfg.split, fallback=fallback)
    prep.pop("zq", None)
    prep.pop("zk", None)
    return bh, prep


def run_preps(cfg, step: int, jobs, workers: int | None = None, merged: bool = False):
    """jobs: iterable of (bh, fallback).  Returns {bh: oracle prologue output}."""
    jobs = list(jobs)
    n = max(1, min(workers or host_cores(), MAX_WORKERS, len(jobs)))
    out = {}
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                             initializer=_init_worker) as ex:
        for f in [ex.submit(prep_job, cfg, step, bh, fb, merged) for bh, fb in jobs]:
            bh, prep = f.result()
            out[bh] = prep
    return out

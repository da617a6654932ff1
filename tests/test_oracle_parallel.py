"""The oracle's process pool (test infrastructure): per-head results from the
pool equal the same oracle functions called directly, for INT4 and FP16
heads, with and without the rotation merged into RoPE, independent of the
number of workers."""
import numpy as np

import oracle as O
from oracle import parallel
from video_diffusion_transformers_amd import synth


def _direct(cfg, bh, rows, fallback, merged=False):
    b, h = divmod(bh, cfg.H)
    q, k, v = synth.head_qkv(cfg, 0, b, h)
    phases = synth.mergeable_phases(cfg.split) if merged else None
    tabs = O.all_rope_tables(cfg.grid, cfg.split, phases=phases)
    r32 = None if merged else synth.rotation_matrices(cfg.split)[1]
    return O.forward_head(q, k, v, tabs, r32, cfg.grid, cfg.split, rows, fallback=fallback)[0]


def test_pool_equals_direct_oracle():
    cfg = synth.custom_config("pool", 1, 3, (2, 9, 17), 128, (44, 42, 42), cfg_seed=71)
    rows = {0: np.arange(cfg.N), 1: np.array([0, 5, 305]), 2: np.arange(0, cfg.N, 7)}
    jobs = [(0, rows[0], False), (1, rows[1], True), (2, rows[2], False)]
    got, secs = parallel.run_heads(cfg, 0, jobs, workers=2)
    for bh, r, fb in jobs:
        assert np.array_equal(got[bh].view(np.uint16), _direct(cfg, bh, r, fb).view(np.uint16))
        assert all(t >= 0 for t in secs[bh])
    one, _ = parallel.run_heads(cfg, 0, jobs[:1], workers=1)
    assert np.array_equal(one[0].view(np.uint16), got[0].view(np.uint16))
    merged, _ = parallel.run_heads(cfg, 0, jobs[2:], workers=1, merged=True)
    assert np.array_equal(merged[2].view(np.uint16),
                          _direct(cfg, 2, rows[2], False, merged=True).view(np.uint16))


def test_pool_prologue_equals_direct():
    cfg = synth.custom_config("pool", 1, 2, (1, 3, 50), 64, (24, 20, 20), cfg_seed=72)
    preps = parallel.run_preps(cfg, 0, [(0, False), (1, True)], workers=2)
    q, k, v = synth.head_qkv(cfg, 0, 0, 0)
    tabs = O.all_rope_tables(cfg.grid, cfg.split)
    r32 = synth.rotation_matrices(cfg.split)[1]
    want = O.prepare_head(q, k, v, tabs, r32, cfg.grid, cfg.split)
    for f in ("q_codes", "k_codes", "v_codes", "q_scale_l2", "k_scale", "v_scale"):
        assert np.array_equal(preps[0][f], want[f]), f
    q1, k1, v1 = synth.head_qkv(cfg, 0, 0, 1)
    want1 = O.prepare_head(q1, k1, v1, tabs, r32, cfg.grid, cfg.split, fallback=True)
    assert np.array_equal(preps[1]["q_rope"].view(np.uint16), want1["q_rope"].view(np.uint16))


def test_literal_recipe_inputs():
    """The literal recipe draws its outlier channels per tensor: Q's and K's
    four heavy channels lie in the temporal partition and differ between Q and
    K of a head (the calibrated recipe shares them)."""
    cfg = synth.CONFIGS["small_lit"]
    q, k, _ = synth.head_qkv(cfg, 0, 0, 0)
    top = lambda x: set(np.argsort(np.abs(x.astype(np.float64)).std(axis=0))[-4:])  # noqa: E731
    tq, tk = top(q), top(k)
    assert all(c < cfg.split[0] for c in tq | tk)
    assert tq != tk
    q2, _, _ = synth.head_qkv(cfg, 1, 0, 0)
    assert top(q2) != tq or not np.array_equal(q2, q)     # fresh per step

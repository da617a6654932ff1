"""The oracle still reproduces the frozen fixtures in tests/golden/ (regression)."""
import os

import numpy as np

import oracle as O
from video_diffusion_transformers_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_thresholds_fixture():
    tau = O.pcode_thresholds()
    rows = _rows("pcode_thresholds.txt")
    assert len(rows) == 15
    for k, bits, _ in rows:
        assert int(np.float32(tau[int(k) - 1]).view(np.uint32)) == int(bits, 16)


def test_kappa_fixture():
    for D, bits, _ in _rows("constants.txt"):
        assert int(np.float32(O.kappa(int(D))).view(np.uint32)) == int(bits, 16)


def test_tiny_output_fixture():
    cfg = synth.CONFIGS["tiny"]
    _, r32 = synth.rotation_matrices(cfg.split)
    tab = O.all_rope_tables(cfg.grid, cfg.split)
    mask = synth.fallback_mask(cfg)
    lines = _rows("tiny_oracle.txt")
    for h in range(cfg.H):
        head = lines[h * (cfg.N + 1)]
        assert head[:2] == ["head", str(h)] and int(head[3]) == mask[h]
        want = np.array([[int(x, 16) for x in ln] for ln in lines[h * (cfg.N + 1) + 1:(h + 1) * (cfg.N + 1)]],
                        np.uint16)
        q, k, v = synth.head_qkv(cfg, 0, 0, h)
        o16, _ = O.forward_head(q, k, v, tab, r32, cfg.grid, cfg.split, np.arange(cfg.N),
                                fallback=bool(mask[h]))
        assert np.array_equal(o16.view(np.uint16), want)

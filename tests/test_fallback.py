"""Fallback-head selection helpers, on CPU tensors with planted errors."""
import numpy as np
import pytest
import torch

from video_diffusion_transformers_amd import fallback


def _planted(B=2, H=5, N=64, D=16, seed=0):
    g = torch.Generator().manual_seed(seed)
    ref = torch.randn(B, H, N, D, generator=g, dtype=torch.float64)
    noise = torch.randn(B, H, N, D, generator=g, dtype=torch.float64)
    levels = torch.tensor([0.0, 1e-3, 0.2, 5e-2, 0.5, 1e-2, 0.3, 0.0, 2e-3, 0.1],
                          dtype=torch.float64).reshape(B, H, 1, 1)
    # noise scaled to exactly `levels` times the reference's norm, head by head
    scale = ref.norm(dim=(2, 3), keepdim=True) / noise.norm(dim=(2, 3), keepdim=True)
    return ref + noise * scale * levels, ref, levels.flatten().numpy()


def test_head_rel_error_recovers_planted_levels():
    test, ref, levels = _planted()
    rel = fallback.head_rel_error(test, ref)
    assert rel.shape == (10,) and rel.dtype == np.float64
    assert np.allclose(rel, levels, rtol=1e-5, atol=1e-7)
    rel16 = fallback.head_rel_error(test.half(), ref.half())
    assert np.allclose(rel16, levels, rtol=2e-2, atol=2e-3)


def test_head_rel_error_rejects_mismatched_shapes():
    a = torch.zeros(1, 2, 4, 8)
    with pytest.raises(ValueError):
        fallback.head_rel_error(a, torch.zeros(1, 2, 4, 4))
    with pytest.raises(ValueError):
        fallback.head_rel_error(a[0], a[0])


def test_worst_heads_mask_and_report():
    _, _, levels = _planted()
    m = fallback.worst_heads_mask(levels, 3)
    assert m.dtype == np.uint8 and list(np.nonzero(m)[0]) == [2, 4, 6]
    assert fallback.worst_heads_mask(levels, 0).sum() == 0
    assert fallback.worst_heads_mask(levels, 10).sum() == 10
    ties = fallback.worst_heads_mask(np.zeros(6), 2)
    assert list(np.nonzero(ties)[0]) == [0, 1]
    with pytest.raises(ValueError):
        fallback.worst_heads_mask(levels, 11)
    r = fallback.report(levels, top=3)
    assert r["worst_heads"] == [[4, 0.5], [6, 0.3], [2, 0.2]]
    assert r["rel_l2_max"] == 0.5 and r["rel_l2_median"] == pytest.approx(np.median(levels))

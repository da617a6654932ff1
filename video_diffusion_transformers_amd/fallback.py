"""Choosing fallback heads from measured error.

RotateAttention keeps accuracy-sensitive units in full precision (RotateAttention
page, Abstract: fallback over attention blocks and denoising steps).  Which
heads are sensitive depends on trained weights, which are not available here;
what can be measured is how far each head's INT4 output lies from a
full-precision output of the same head.  These helpers turn two outputs of the
same inputs (INT4 attention of every head, and FP16 attention of every head,
both from the HIP kernels) into a per-head relative error and a fallback mask
that sends the worst heads to FP16.  They read finished outputs only and are no
step of the forward pass.
"""
from __future__ import annotations

import numpy as np


def head_rel_error(o_test, o_ref) -> np.ndarray:
    """Per-head relative L2 distance ||o_test - o_ref|| / ||o_ref|| over each
    head's whole [N, D] output.  Both are torch tensors [B, H, N, D] (any
    device, any float dtype); accumulation is in float32 on their device,
    the result a float64 array [B*H]."""
    if tuple(o_test.shape) != tuple(o_ref.shape) or o_test.dim() != 4:
        raise ValueError(f"outputs must share one [B, H, N, D] shape: "
                         f"{tuple(o_test.shape)} vs {tuple(o_ref.shape)}")
    B, H = o_test.shape[:2]
    a = o_test.float().reshape(B * H, -1)
    b = o_ref.float().reshape(B * H, -1)
    num = (a - b).square().sum(dim=1).sqrt()
    den = b.square().sum(dim=1).sqrt().clamp_min(1e-30)
    return (num / den).double().cpu().numpy()


def worst_heads_mask(rel: np.ndarray, count: int) -> np.ndarray:
    """uint8 [B*H] mask with the `count` largest errors set (ties: lower
    head index first).  It is a valid fallback mask for every entry point."""
    rel = np.asarray(rel, np.float64)
    if not 0 <= count <= rel.size:
        raise ValueError(f"count {count} outside [0, {rel.size}]")
    order = np.lexsort((np.arange(rel.size), -rel))
    mask = np.zeros(rel.size, np.uint8)
    mask[order[:count]] = 1
    return mask


def report(rel: np.ndarray, top: int = 5) -> dict:
    """Summary of a per-head error array: median, max and the worst heads."""
    rel = np.asarray(rel, np.float64)
    worst = np.nonzero(worst_heads_mask(rel, min(top, rel.size)))[0]
    worst = worst[np.argsort(-rel[worst], kind="stable")]
    return {"rel_l2_median": round(float(np.median(rel)), 6),
            "rel_l2_max": round(float(rel.max()), 6),
            "worst_heads": [[int(h), round(float(rel[h]), 6)] for h in worst]}

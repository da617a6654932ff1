"""Shared helpers for the GPU parity tests: inputs on the device, the HIP path
through the C ABI, and the oracle on the same seeded inputs."""
from __future__ import annotations

import functools

import numpy as np

import oracle as O
from video_diffusion_transformers_amd import synth

TOL = 2e-3   # max|O_gpu - O_oracle| <= TOL * max|O_oracle| on fp16 outputs


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def pack_rows(codes: np.ndarray) -> np.ndarray:
    """INT4 codes [n, D] -> packed bytes [n, D/2] in the documented nibble layout:
    byte i of each 8-element group holds element i (low nibble) and i+4 (high)."""
    n, D = codes.shape
    c = (codes.astype(np.int16) & 0xF).astype(np.uint8).reshape(n, D // 8, 8)
    return (c[:, :, :4] | (c[:, :, 4:] << 4)).reshape(n, D // 2)


def pack_vt_blocks(codes: np.ndarray, N_pad: int) -> np.ndarray:
    """V codes [N, D] -> [NB, D, 64]: per 128-token block, transposed, packed along keys."""
    N, D = codes.shape
    full = np.zeros((N_pad, D), np.int8)
    full[:N] = codes
    out = []
    for b in range(N_pad // 128):
        out.append(pack_rows(np.ascontiguousarray(full[b * 128:(b + 1) * 128].T)))
    return np.stack(out)


class Run:
    """One config on the device: inputs, RoPE/rotation, prepared buffers."""

    def __init__(self, cfg: synth.Config, step: int = 0):
        torch = torch_cuda()
        from video_diffusion_transformers_amd import rotattn as R
        self.R = R
        self.cfg = cfg
        self.step = step
        self.shape = R.shape_of(cfg)
        self.NB = R.n_blocks(self.shape)
        self.N_pad = self.NB * 128
        q, k, v = synth.all_heads_qkv(cfg, step)
        self.host = (q, k, v)
        self.q, self.k, self.v = (torch.from_numpy(x).cuda() for x in (q, k, v))
        self.r64, self.r32 = synth.rotation_matrices(cfg.split)
        self.rr = R.RopeRotDevice(self.shape, self.r32)
        self.mask = synth.fallback_mask(cfg)
        self.prep = R.PreparedDevice(self.shape, with_rope=True)

    def prepare(self, mask="cfg"):
        m = self.mask if isinstance(mask, str) else mask
        self.R.prepare_qkv(self.shape, self.q, self.k, self.v, self.rr, self.prep, m)

    def gpu_prepared(self):
        """Host copies of the prepared buffers, shaped per head."""
        torch = torch_cuda()
        torch.cuda.synchronize()
        BH, D, NB, N = self.cfg.BH, self.cfg.D, self.NB, self.cfg.N
        p = self.prep
        out = {
            "q4": p.view("q4", torch.uint8, BH * self.N_pad * D // 2).cpu().numpy().reshape(BH, self.N_pad, D // 2),
            "k4": p.view("k4", torch.uint8, BH * self.N_pad * D // 2).cpu().numpy().reshape(BH, self.N_pad, D // 2),
            "v4": p.view("v4", torch.uint8, BH * NB * D * 64).cpu().numpy().reshape(BH, NB, D, 64),
        }
        for f in ("q_scale_l2", "k_scale", "v_scale"):
            out[f] = p.view(f, torch.float32, BH * NB).cpu().numpy().reshape(BH, NB)
        for f in ("q_rope", "k_rope"):
            out[f] = p.view(f, torch.int16, BH * N * D).cpu().numpy().view(np.uint16).reshape(BH, N, D)
        return out

    def empty_out(self):
        torch = torch_cuda()
        return torch.zeros((self.cfg.B, self.cfg.H, self.cfg.N, self.cfg.D), dtype=torch.float16,
                           device="cuda")

    @functools.cached_property
    def tables(self):
        return O.all_rope_tables(self.cfg.grid, self.cfg.split)

    @functools.lru_cache(maxsize=64)
    def oracle_prep(self, bh: int, fallback: bool = False):
        q, k, v = (x.reshape(self.cfg.BH, self.cfg.N, self.cfg.D)[bh] for x in self.host)
        return O.prepare_head(q, k, v, self.tables, self.r32, self.cfg.grid, self.cfg.split,
                              fallback=fallback)

    def oracle_int4(self, bh: int, rows, record=None):
        p = self.oracle_prep(bh)
        return O.int4_attention(p["q_codes"], p["q_scale_l2"], p["k_codes"], p["k_scale"],
                                p["v_codes"], p["v_scale"], rows, record=record)

    def oracle_fp16(self, bh: int, rows):
        p = self.oracle_prep(bh, fallback=True)
        v = self.host[2].reshape(self.cfg.BH, self.cfg.N, self.cfg.D)[bh]
        return O.fp16_attention(p["q_rope"], p["k_rope"], v, rows)


def check_out(o_gpu: np.ndarray, o_ref16: np.ndarray, what: str):
    ref = o_ref16.astype(np.float64)
    err = np.abs(o_gpu.astype(np.float64) - ref).max()
    scale = np.abs(ref).max()
    assert np.all(np.isfinite(o_gpu)), what
    assert err <= TOL * scale, f"{what}: max-abs {err:.3g} > {TOL} * max|O| {scale:.3g}"
    return err / scale

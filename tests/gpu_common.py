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


E4M3 = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E}


def fp8_bytes(codes: np.ndarray) -> np.ndarray:
    """INT4 codes -> FP8 E4M3 bytes of the integers (the FP8 layout)."""
    mag = np.abs(codes.astype(np.int16))
    lut = np.array([E4M3[i] for i in range(8)], np.uint8)
    return lut[mag] | np.where(codes < 0, 0x80, 0).astype(np.uint8)


def fp8_vt_blocks(codes: np.ndarray, N_pad: int) -> np.ndarray:
    """V codes [N, D] -> [NB, D, 128] FP8 bytes: per 128-token block, transposed,
    each 64-key half in the P.V operand order (byte 32h + j holds key
    32h + 8((j%16)/4) + 4(j/16) + j%4)."""
    N, D = codes.shape
    full = np.zeros((N_pad, D), np.int8)
    full[:N] = codes
    perm = np.empty(128, np.int64)
    for c in range(2):
        for h in range(2):
            for j in range(32):
                perm[64 * c + 32 * h + j] = 64 * c + 32 * h + 8 * ((j % 16) // 4) + 4 * (j // 16) + j % 4
    assert sorted(perm) == list(range(128))
    out = []
    for b in range(N_pad // 128):
        blk = full[b * 128:(b + 1) * 128]          # [128 keys, D]
        out.append(fp8_bytes(blk[perm].T))          # [D, 128]
    return np.stack(out)


def _e2m3_value(bits: int) -> float:
    """Value of a 6-bit FP6 E2M3 pattern: sign bit 5, exponent bits 4-3 (bias
    1, 0 = subnormal), mantissa bits 2-0."""
    s, e, m = bits >> 5, (bits >> 3) & 3, bits & 7
    mag = m / 8 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8)
    return -mag if s else mag


# code -> E2M3 bits, found by search over the 64 patterns (+0 for code 0)
E2M3 = {c: min(b for b in range(64) if _e2m3_value(b) == c) for c in range(-7, 8)}


def _pack_fields(fields: np.ndarray) -> np.ndarray:
    """[..., 32] six-bit fields -> [..., 32] bytes: field k in bits 6k..6k+5 of
    the first 24 bytes (little-endian), then 8 zero bytes."""
    bits = ((fields[..., :, None].astype(np.uint8) >> np.arange(6, dtype=np.uint8)) & 1)
    bits = bits.reshape(*fields.shape[:-1], 192)
    packed = np.packbits(bits, axis=-1, bitorder="little")          # [..., 24]
    pad = np.zeros((*fields.shape[:-1], 8), np.uint8)
    return np.concatenate([packed, pad], axis=-1)


def fp6_rows(codes: np.ndarray) -> np.ndarray:
    """Q/K codes [n, D] -> the FP6 layout's rows [n, D]: per 32-channel group,
    channel 32g + k in field k."""
    n, D = codes.shape
    lut = np.array([E2M3[c] for c in range(-7, 8)], np.uint8)
    f = lut[codes.astype(np.int16) + 7].reshape(n, D // 32, 32)
    return _pack_fields(f).reshape(n, D)


def fp6_vt_blocks(codes: np.ndarray, N_pad: int) -> np.ndarray:
    """V codes [N, D] -> [NB, D, 128] FP6 layout: per 128-token block, row d in
    groups g = 2c + h whose field k holds key 64c + 32(k/16) + 8((k%16)/4) +
    4h + k%4."""
    N, D = codes.shape
    full = np.zeros((N_pad, D), np.int16)
    full[:N] = codes
    lut = np.array([E2M3[c] for c in range(-7, 8)], np.uint8)
    keys = np.array([[64 * (g // 2) + 32 * (k // 16) + 8 * ((k % 16) // 4) + 4 * (g % 2) + k % 4
                      for k in range(32)] for g in range(4)])
    assert sorted(keys.ravel()) == list(range(128))
    out = []
    for b in range(N_pad // 128):
        blk = full[b * 128:(b + 1) * 128]                # [128 keys, D]
        f = lut[blk[keys] + 7]                           # [4, 32, D]
        out.append(_pack_fields(f.transpose(2, 0, 1)).reshape(D, 128))
    return np.stack(out)


def code_rows(codes: np.ndarray, layout: str) -> np.ndarray:
    """Q/K codes in the bytes of a prepared layout ("packed", "fp8", "fp6")."""
    return {"packed": pack_rows, "fp8": fp8_bytes, "fp6": fp6_rows}[layout](codes)


def v_blocks(codes: np.ndarray, N_pad: int, layout: str) -> np.ndarray:
    return {"packed": pack_vt_blocks, "fp8": fp8_vt_blocks, "fp6": fp6_vt_blocks}[layout](codes, N_pad)


def fp16_vt_tiles(v: np.ndarray, N_pad: int) -> np.ndarray:
    """fp16 V [N, D] -> [N_pad/64, D, 64] V^T tiles in the fp16 P.V operand
    order: position 32s + 4c + i holds key 32s + 4c' + i, c' = c with bits 0
    and 1 swapped; keys >= N zero (bit patterns as uint16)."""
    N, D = v.shape
    full = np.zeros((N_pad, D), np.uint16)
    full[:N] = v.view(np.uint16)
    perm = np.empty(64, np.int64)
    for pos in range(64):
        s_, pc, i = pos // 32, (pos % 32) // 4, pos % 4
        c = (pc & 4) | ((pc & 1) << 1) | ((pc >> 1) & 1)
        perm[pos] = 32 * s_ + 4 * c + i
    assert sorted(perm) == list(range(64))
    return np.stack([full[64 * t:64 * (t + 1)][perm].T for t in range(N_pad // 64)])


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

    def __init__(self, cfg: synth.Config, step: int = 0, layout: int = 2, merged: bool = False,
                 qkv=None):
        """merged: the rotation is merged into the RoPE tables (seeded pair
        phases, no dense rotation matrices).  qkv: host fp16 Q, K, V
        [B][H][N][D] to use instead of the workload's seeded ones."""
        torch = torch_cuda()
        from video_diffusion_transformers_amd import rotattn as R
        self.R = R
        self.cfg = cfg
        self.step = step
        self.shape = R.shape_of(cfg)
        self.NB = R.n_blocks(self.shape)
        self.N_pad = self.NB * 128
        q, k, v = synth.all_heads_qkv(cfg, step) if qkv is None else qkv
        self.host = (q, k, v)
        self.q, self.k, self.v = (torch.from_numpy(x).cuda() for x in (q, k, v))
        self.merged = merged
        self.phases = synth.mergeable_phases(cfg.split) if merged else None
        if merged:
            self.r64 = self.r32 = None
        else:
            self.r64, self.r32 = synth.rotation_matrices(cfg.split)
        self.rr = R.RopeRotDevice(self.shape, self.r32, phases=self.phases)
        self.mask = synth.fallback_mask(cfg)
        self.layout = layout
        self.prep = R.PreparedDevice(self.shape, with_rope=True, layout=layout)

    def prepare(self, mask="cfg"):
        m = self.mask if isinstance(mask, str) else mask
        self.R.prepare_qkv(self.shape, self.q, self.k, self.v, self.rr, self.prep, m)

    def gpu_prepared(self):
        """Host copies of the prepared buffers, shaped per head."""
        torch = torch_cuda()
        torch.cuda.synchronize()
        BH, D, NB, N = self.cfg.BH, self.cfg.D, self.NB, self.cfg.N
        p = self.prep
        byte = self.layout in (self.R.LAYOUT_FP8, self.R.LAYOUT_FP6)  # one byte per code
        w = D if byte else D // 2      # bytes per code row
        vw = 128 if byte else 64
        out = {
            "q4": p.view("q4", torch.uint8, BH * self.N_pad * w).cpu().numpy().reshape(BH, self.N_pad, w),
            "k4": p.view("k4", torch.uint8, BH * self.N_pad * w).cpu().numpy().reshape(BH, self.N_pad, w),
            "v4": p.view("v4", torch.uint8, BH * NB * D * vw).cpu().numpy().reshape(BH, NB, D, vw),
        }
        for f in ("q_scale_l2", "k_scale", "v_scale"):
            out[f] = p.view(f, torch.float32, BH * NB).cpu().numpy().reshape(BH, NB)
        for f in ("q_rope", "k_rope"):
            out[f] = (p.view(f, torch.int16, BH * self.N_pad * D).cpu().numpy().view(np.uint16)
                      .reshape(BH, self.N_pad, D))
        out["v_t"] = (p.view("v_t", torch.int16, BH * self.N_pad * D).cpu().numpy().view(np.uint16)
                      .reshape(BH, self.N_pad // 64, D, 64))
        return out

    def empty_out(self):
        torch = torch_cuda()
        return torch.zeros((self.cfg.B, self.cfg.H, self.cfg.N, self.cfg.D), dtype=torch.float16,
                           device="cuda")

    @functools.cached_property
    def tables(self):
        return O.all_rope_tables(self.cfg.grid, self.cfg.split, phases=self.phases)

    @functools.lru_cache(maxsize=64)
    def oracle_prep(self, bh: int, fallback: bool = False):
        q, k, v = (x.reshape(self.cfg.BH, self.cfg.N, self.cfg.D)[bh] for x in self.host)
        return O.prepare_head(q, k, v, self.tables, self.r32, self.cfg.grid, self.cfg.split,
                              fallback=fallback)

    def oracle_int4(self, bh: int, rows, record=None, normalizer="exp"):
        p = self.oracle_prep(bh)
        return O.int4_attention(p["q_codes"], p["q_scale_l2"], p["k_codes"], p["k_scale"],
                                p["v_codes"], p["v_scale"], rows, record=record,
                                normalizer=normalizer)

    def oracle_fp16(self, bh: int, rows):
        p = self.oracle_prep(bh, fallback=True)
        v = self.host[2].reshape(self.cfg.BH, self.cfg.N, self.cfg.D)[bh]
        return O.fp16_attention(p["q_rope"], p["k_rope"], v, rows)


def check_prologue_heads(run, heads, layout: str, preps):
    """The prepared buffers of `run` for the given heads against the oracle's
    prologue outputs `preps` {bh: prepare_head(...)}: codes in the bytes of
    `layout` and scale bits of INT4 heads; RoPE'd Q'/K' and V^T tiles of
    fallback heads; bit for bit."""
    name = run.cfg.name
    g = run.gpu_prepared()
    for bh in heads:
        fb = bool(run.mask[bh])
        p = preps[bh]
        if fb:
            N = run.cfg.N
            for t in ("q", "k"):
                assert np.array_equal(g[f"{t}_rope"][bh][:N], p[f"{t}_rope"].view(np.uint16))
                assert not g[f"{t}_rope"][bh][N:].any()
            v = run.host[2].reshape(run.cfg.BH, N, run.cfg.D)[bh]
            assert np.array_equal(g["v_t"][bh], fp16_vt_tiles(v, run.N_pad)), (name, bh, "v_t")
            continue
        for t in ("q", "k"):
            rows = code_rows(p[f"{t}_codes"], layout)
            want = np.zeros((run.N_pad, rows.shape[1]), np.uint8)
            want[:run.cfg.N] = rows
            assert np.array_equal(g[f"{t}4"][bh], want), (name, bh, t)
        assert np.array_equal(g["v4"][bh], v_blocks(p["v_codes"], run.N_pad, layout)), (name, bh)
        for f in ("q_scale_l2", "k_scale", "v_scale"):
            assert np.array_equal(g[f][bh].view(np.uint32), p[f].view(np.uint32)), (name, bh, f)


def check_out(o_gpu: np.ndarray, o_ref16: np.ndarray, what: str):
    """max|O_gpu - O_oracle| <= TOL * max|O_oracle|; an all-zero reference
    (zero V) must be matched exactly."""
    ref = o_ref16.astype(np.float64)
    err = np.abs(o_gpu.astype(np.float64) - ref).max()
    scale = np.abs(ref).max()
    assert np.all(np.isfinite(o_gpu)), what
    assert err <= TOL * scale, f"{what}: max-abs {err:.3g} > {TOL} * max|O| {scale:.3g}"
    return err / scale if scale > 0 else 0.0


_POOL_CACHE = {}


def pool_reference(cfg, step, jobs, normalizer="exp", merged=False):
    """Oracle output rows of many heads, computed in a process pool over the
    host's cores (each worker regenerates its head from the seeds); cached per
    workload and job list.  jobs: [(bh, rows, fallback)]."""
    from oracle import parallel
    key = (cfg, step, normalizer, merged,
           tuple((bh, np.asarray(rows).tobytes(), bool(fb)) for bh, rows, fb in jobs))
    if key not in _POOL_CACHE:
        _POOL_CACHE.clear()
        _POOL_CACHE[key] = parallel.run_heads(cfg, step, jobs, normalizer=normalizer,
                                              merged=merged)[0]
    return _POOL_CACHE[key]

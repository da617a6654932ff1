"""Benchmark: RotateAttention INT4 FlashAttention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload 720p]

A step is one pass of the whole hot path over one batch of synthetic inputs
that are already resident in HBM: the prologue (3D RoPE + partition-wise
rotation + INT4 quantize/pack), the INT4 attention over the INT4 heads and
the FP16 FlashAttention over the fallback heads -- the launch sequence of
rotattn_mixed_fwd.  The headline workload is the 720p-shaped one (B=1, H=40,
grid 21x45x80, N=75600, D=128, all heads INT4).  The metric is effective
attention TOPS = 4*B*H*N^2*D / step time.

Prints one JSON line.  Besides the contract fields it carries the roofline
of the dominant kernel (the INT4 attention on the FP6 layout, timed with HIP
events on the stream it runs on, with the VALU-busy share of the unit that
bounds it), the same for the FP8-layout and i8-MFMA implementations of that
kernel, the per-kernel times, the
Mixed workload (4 denoising steps, a fixed seeded quarter of the heads in
FP16, fresh inputs per step), the 480p workload, a synthetic DiT block, and
the CPU oracle timed on a bounded sample on this host's cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TOPS at 1 MI355X + % of i8 MFMA peak, N=75600 D=128"
PEAK_I8_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POPS); dense fp8 is the same
PEAK_FP6_TOPS = 10100.0      # MI355X dense fp6 MFMA (10.1 POPS)
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA (2.5 PFLOPS)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (8 TB/s)
PMC_FILE = os.path.join(ROOT, "profiles", "int4_attn_fp6_720p_pmc.txt")
SQ_FILE = os.path.join(ROOT, "profiles", "int4_attn_fp6_720p_sq_counters.txt")
PROFILED_WORKLOAD = "720p"   # the workload both counter summaries were taken on
KERNEL_SRC = os.path.join(ROOT, "video_diffusion_transformers_amd", "csrc", "int4_attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p", choices=["720p", "480p", "small", "mixed"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only: skip the packed-layout, mixed_fwd and all-FP16 "
                         "side figures (used for counter collection)")
    ap.add_argument("--mixed-steps", type=int, default=4,
                    help="denoising steps of the mixed workload to time as a side figure (0: skip)")
    return ap.parse_args()


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the INT4 kernel from the committed rocprofv3
    counter summary, if it was taken on this workload and the current kernel
    source."""
    if workload != PROFILED_WORKLOAD or not os.path.exists(PMC_FILE):
        return None
    vals = {}
    with open(PMC_FILE) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def valu_busy_from_profile(workload: str):
    """Share of the INT4 kernel's SIMD clocks with a VALU instruction issuing,
    from the committed rocprofv3 SQ counter summary, if it was taken on this
    workload and the current kernel source (the kernel is bound by that VALU
    work, not by MFMA)."""
    if workload != PROFILED_WORKLOAD or not os.path.exists(SQ_FILE):
        return None
    with open(SQ_FILE) as f:
        txt = f.read()
    if f"int4_attn.hip sha256[:16] = {kernel_hash()}" not in txt:
        return None
    for ln in txt.splitlines():
        if ln.startswith("VALU share of SIMD clocks:"):
            try:
                return float(ln.split(":", 1)[1])
            except ValueError:
                return None
    return None


def prologue_bytes(BH: int, N: int, D: int):
    """Algorithmic HBM bytes of the prologue (per token and head: read Q, K, V
    fp16, write Q, K, V as INT4 codes, two per byte; block scales are
    negligible) and the bytes its FP6 layout actually writes (one byte per
    code: 32 six-bit codes and 8 pad bytes per 32 bytes)."""
    algorithmic = BH * N * (3 * 2 * D + 3 * D // 2)
    layout = BH * N * (3 * 2 * D + 3 * D)
    return algorithmic, layout


def time_calls(fn, reps: int) -> float:
    """Mean ms of fn() over reps calls (HIP events on torch's current stream,
    the stream the library enqueues on), after one untimed call."""
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the INT4 "
              f"attention shards by head with no exchange inside the kernel, so a multi-GPU run "
              f"is one GPU's run per shard; it is not provided.", file=sys.stderr)
        sys.exit(2)

    import torch
    from video_diffusion_transformers_amd import rotattn as R
    from video_diffusion_transformers_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = synth.CONFIGS[args.workload]
    shape = R.shape_of(cfg)
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    ops = 4.0 * B * H * N * N * D

    t0 = time.time()
    q, k, v = synth.all_heads_qkv(cfg, 0)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    _, r32 = synth.rotation_matrices(cfg.split)
    rr = R.RopeRotDevice(shape, r32)
    mask = synth.fallback_mask(cfg)
    prep = R.PreparedDevice(shape, with_rope=True, layout=R.LAYOUT_FP6)
    o = torch.empty((B, H, N, D), dtype=torch.float16, device="cuda")
    BH = B * H
    n_fb = int(mask.sum())
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s: {cfg.name} B={B} H={H} N={N} D={D} "
          f"fallback heads={n_fb}", file=sys.stderr, flush=True)

    def step(ev=None):
        if ev: ev[0].record()
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, mask)
        if ev: ev[1].record()
        R.int4_fwd(shape, prep, o, mask=mask)
        if ev: ev[2].record()
        if n_fb:
            R.fp16_fwd_prepared(shape, prep, o, head_select=mask)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    k1 = np.array([e[0].elapsed_time(e[1]) for e in evs])
    k2 = np.array([e[1].elapsed_time(e[2]) for e in evs])
    k3 = np.array([e[2].elapsed_time(e[3]) for e in evs])
    tot = np.array([e[0].elapsed_time(e[3]) for e in evs])
    ms_per_step = float(wall_ms)
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step "
          f"(prologue {k1.mean():.3f}, int4 {k2.mean():.3f}, fp16 {k3.mean():.3f} ms)",
          file=sys.stderr, flush=True)

    n_int4 = BH - n_fb
    int4_ops = 4.0 * n_int4 * N * N * D
    k2_ms = float(k2.mean())
    achieved = int4_ops / (k2_ms * 1e-3) / 1e12 if n_int4 else 0.0
    traffic = traffic_from_profile(args.workload)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP6_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_FP6_TOPS, 4), "traffic": traffic,
                "kernel": "k_int4_attn_f8<128, false, false, true> (FP6 layout)",
                "operands": "INT4 codes as FP6 E2M3 (Q, K, V) and P codes as FP6 E2M3 "
                            "(code/2), both MFMA operands FP6; fp32 accumulation exact on these "
                            "integers; priced against the dense fp6 peak",
                "frac_of_i8_fp8_peak": round(achieved / PEAK_I8_TOPS, 4),
                "algorithmic_ops_per_launch": int4_ops,
                "limiter": "valu", "limiter_busy": valu_busy_from_profile(args.workload)}
    k1_ms = float(k1.mean())
    pro_alg, pro_layout = prologue_bytes(BH, N, D)
    kernels = {
        "prologue_ms": round(k1_ms, 4),
        "prologue_hbm_frac": round(pro_alg / (k1_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "prologue_algorithmic_bytes": pro_alg,
        "prologue_layout_bytes": pro_layout,
        "prologue_layout_bytes_frac": round(pro_layout / (k1_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "int4_attn_ms": round(k2_ms, 4),
        "int4_attn_ms_min": round(float(k2.min()), 4),
        "int4_attn_i8_peak_frac": round(achieved / PEAK_I8_TOPS, 4),
        "fp16_attn_ms": round(float(k3.mean()), 4),
        "event_step_ms": round(float(tot.mean()), 4),
    }
    roofline_i8 = roofline_f8 = None

    if not args.no_extras:
        # the same INT4 attention on the FP8 layout: Q, K, V codes as E4M3, P as
        # FP6 (FP8 x FP6 runs at the FP8 rate)
        prep_8 = R.PreparedDevice(shape, with_rope=n_fb > 0, layout=R.LAYOUT_FP8)
        R.prepare_qkv(shape, qd, kd, vd, rr, prep_8, mask)
        f8_ms = time_calls(lambda: R.int4_fwd(shape, prep_8, o, mask=mask), 3)
        del prep_8
        f8_ach = int4_ops / (f8_ms * 1e-3) / 1e12 if n_int4 else 0.0
        roofline_f8 = {"bound": "mfma", "achieved": round(f8_ach, 2), "peak": PEAK_I8_TOPS,
                       "unit": "TOP/s", "frac": round(f8_ach / PEAK_I8_TOPS, 4), "traffic": None,
                       "kernel": "k_int4_attn_f8<128, false, false, false> (FP8 layout)",
                       "operands": "INT4 codes as FP8 E4M3 (Q, K, V), P codes as FP6 E2M3 "
                                   "(code/2); FP8 x FP6 runs at the FP8 rate, whose dense peak "
                                   "equals the i8 one",
                       "ms": round(f8_ms, 4), "algorithmic_ops_per_launch": int4_ops}
        kernels["int4_attn_fp8_layout_ms"] = round(f8_ms, 4)
        print(f"[bench] FP8-layout kernel {f8_ms:.3f} ms", file=sys.stderr, flush=True)

        # the same INT4 attention on the nibble-packed layout: int8 lanes on the
        # i8 MFMA with int32 accumulation (fallback heads, if any, need the
        # fp16 RoPE'd buffers as well)
        prep_p = R.PreparedDevice(shape, with_rope=n_fb > 0, layout=R.LAYOUT_PACKED)
        R.prepare_qkv(shape, qd, kd, vd, rr, prep_p, mask)
        i8_ms = time_calls(lambda: R.int4_fwd(shape, prep_p, o, mask=mask), 3)
        del prep_p
        i8_ach = int4_ops / (i8_ms * 1e-3) / 1e12 if n_int4 else 0.0
        roofline_i8 = {"bound": "mfma", "achieved": round(i8_ach, 2), "peak": PEAK_I8_TOPS,
                       "unit": "TOP/s", "frac": round(i8_ach / PEAK_I8_TOPS, 4), "traffic": None,
                       "kernel": "k_int4_attn<128>",
                       "operands": "INT4 codes unpacked to int8 lanes, v_mfma_i32_32x32x32_i8 "
                                   "with int32 accumulation",
                       "ms": round(i8_ms, 4), "algorithmic_ops_per_launch": int4_ops}
        kernels["int4_attn_packed_i8_ms"] = round(i8_ms, 4)
        print(f"[bench] i8-MFMA kernel {i8_ms:.3f} ms", file=sys.stderr, flush=True)

        # mixed_fwd (one C call) on the same inputs, as a cross-check of the sequence
        ws = torch.empty(R.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        kernels["mixed_fwd_call_ms"] = round(
            time_calls(lambda: R.mixed_fwd(shape, qd, kd, vd, rr, mask, ws, o), 3), 4)
        del ws

        # INT4 output of every head, kept for the per-head error report below
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, None)
        R.int4_fwd(shape, prep, o, mask=None)
        o_int4 = o.clone()

        # FP16 FlashAttention on every head of the same shape (kernel-level analogue
        # of the full-precision baseline) -- context figure
        all_fb = np.ones(BH, np.uint8)
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, all_fb)
        f16_ms = time_calls(lambda: R.fp16_fwd_prepared(shape, prep, o, head_select=all_fb), 1)
        kernels["fp16_attn_all_heads_ms"] = round(f16_ms, 4)
        kernels["fp16_attn_f16_peak_frac"] = round(ops / (f16_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)
        kernels["int4_vs_fp16_kernel_speedup"] = round(f16_ms / k2_ms, 3) if n_int4 == BH else None
        print(f"[bench] fp16 all heads {f16_ms:.3f} ms", file=sys.stderr, flush=True)
        from video_diffusion_transformers_amd import fallback
        kernels["int4_vs_fp16_head_error"] = dict(
            reference="FP16 attention kernel, same inputs",
            **fallback.report(fallback.head_rel_error(o_int4, o)))

        # the FP16 attention on caller tensors (staging into a workspace, then
        # the same kernel): the RoPE'd fp16 Q'/K' of the prologue's buffers
        # stand in for a caller's, V is the input
        ws16 = torch.empty(R.fp16_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        qv = prep.view("q_rope", torch.float16, BH * R.n_blocks(shape) * 128 * D)
        kv = prep.view("k_rope", torch.float16, BH * R.n_blocks(shape) * 128 * D)
        qr = qv.view(BH, -1, D)[:, :N].reshape(B, H, N, D).contiguous()
        kr = kv.view(BH, -1, D)[:, :N].reshape(B, H, N, D).contiguous()
        o2 = torch.empty_like(o)
        kernels["fp16_fwd_caller_buffers_ms"] = round(
            time_calls(lambda: R.fp16_fwd(shape, qr, kr, vd, o2, ws16), 1), 4)
        del ws16, qr, kr, o2

        # the rotation merged into RoPE (seeded pair phases in the tables, no
        # dense rotation): prologue time and the same error report
        rr_m = R.RopeRotDevice(shape, None, phases=synth.mergeable_phases(cfg.split))
        kernels["prologue_merged_rotation_ms"] = round(
            time_calls(lambda: R.prepare_qkv(shape, qd, kd, vd, rr_m, prep, None), 3), 4)
        R.int4_fwd(shape, prep, o_int4, mask=None)
        kernels["int4_merged_rotation_vs_fp16_head_error"] = dict(
            reference="FP16 attention kernel, same inputs",
            **fallback.report(fallback.head_rel_error(o_int4, o)))
        print(f"[bench] prologue with the rotation merged into RoPE "
              f"{kernels['prologue_merged_rotation_ms']:.3f} ms", file=sys.stderr, flush=True)
        del o_int4, rr_m
    del qd, kd, vd, prep, o
    torch.cuda.empty_cache()

    dit = None
    if not args.no_extras and args.workload == "720p":
        dit = bench_dit_block(cfg)
    mixed = None
    if args.mixed_steps and args.workload == "720p":
        mixed = bench_mixed(args.mixed_steps)
    p480 = None
    if not args.no_extras and args.workload == "720p":
        p480 = bench_workload("480p")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, ops)

    value = ops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} H={H} grid {'x'.join(map(str, cfg.grid))} "
                               f"N={N} D={D} split {'/'.join(map(str, cfg.split))}, "
                               f"{BH - n_fb} INT4 heads + {n_fb} FP16 heads, seeded synthetic "
                               f"fp16 Q/K/V (per-channel lognormal scales with 4 temporal "
                               f"outlier channels x10-30, Q and K scaled to a 2.5-nat logit "
                               f"spread; sparse x15 V token outliers)",
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": D,
                   "parallelism": "single GPU"},
        "percent_i8_peak_step": round(100 * value / PEAK_I8_TOPS, 2),
        "roofline": roofline,
        "roofline_fp8_layout_kernel": roofline_f8,
        "roofline_i8_mfma_kernel": roofline_i8,
        "kernels": kernels,
        "mixed": mixed,
        "workload_480p": p480,
        "dit_block": dit,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_dit_block(cfg, width: int = 5120, reps: int = 2):
    """Side figure: a synthetic DiT self-attention block at the 720p shape with
    model width 5120 (40 heads x 128): QKV projection GEMM, attention, output
    projection GEMM (fp16 GEMMs on hipBLASLt, seeded random weights).  INT4
    attention with the prologue reading the projection's token-major output in
    place and O written token-major, against the same block with contiguous
    copies around the attention, against the library's own QKV projection with
    the prologue as its epilogue, and against FP16 attention on every head."""
    import torch
    from video_diffusion_transformers_amd import dit_block, rotattn as R, synth
    shape = R.shape_of(cfg)
    _, r32 = synth.rotation_matrices(cfg.split)
    blk = dit_block.DiTAttentionBlock(shape, width, R.RopeRotDevice(shape, r32), seed=5)
    g = torch.Generator(device="cpu").manual_seed(6)
    x = torch.randn(cfg.B, cfg.N, width, generator=g).half().cuda()
    res = {}
    for key, kw in (("int4_fused_ms", dict(fp16=False, fused=True)),
                    ("int4_unfused_ms", dict(fp16=False, fused=False)),
                    ("int4_gemm_prologue_ms", dict(fp16=False, gemm_prologue=True)),
                    ("fp16_fused_ms", dict(fp16=True, fused=True))):
        blk.forward(x, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            blk.forward(x, **kw)
        e1.record()
        torch.cuda.synchronize()
        res[key] = round(e0.elapsed_time(e1) / reps, 3)
    # the projections alone
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(x, blk.w_qkv, out=blk.qkv)
        torch.matmul(blk.o_tok.view(cfg.B, cfg.N, -1), blk.w_o)
    e1.record()
    torch.cuda.synchronize()
    res["projections_ms"] = round(e0.elapsed_time(e1) / reps, 3)
    # the QKV projection + prologue: hipBLASLt GEMM then the prologue on its
    # token-major output, against the one fused launch
    q, k, v = blk.qkv.view(cfg.B, cfg.N, 3, cfg.H, cfg.D).permute(2, 0, 3, 1, 4)
    res["qkv_gemm_ms"] = round(time_calls(lambda: torch.matmul(x, blk.w_qkv, out=blk.qkv), reps), 3)
    res["prologue_strided_ms"] = round(
        time_calls(lambda: R.prepare_qkv(shape, q, k, v, blk.rr, blk.prep), reps), 3)
    res["qkv_gemm_prologue_fused_ms"] = round(
        time_calls(lambda: R.qkv_proj_prepare(shape, x, blk.w_qkv_rows, None, blk.rr, blk.prep),
                   reps), 3)
    res["int4_vs_fp16_block_speedup"] = round(res["fp16_fused_ms"] / res["int4_fused_ms"], 3)
    print(f"[bench] DiT block: {res}", file=sys.stderr, flush=True)
    del blk, x
    torch.cuda.empty_cache()
    return dict(workload=f"720p shape, width {width}, QKV projection + attention + output "
                         f"projection, random weights (timing only)", **res)


def bench_mixed(steps: int):
    """The Mixed workload: 720p shape, a seeded mask sending 10 of 40 heads to
    the FP16 attention, fixed across steps, and one rotattn_mixed_fwd per
    denoising step with fresh seeded Q/K/V.  Each step is timed as one call
    (HIP events) after an untimed call on the same inputs."""
    import torch
    from video_diffusion_transformers_amd import rotattn as R
    from video_diffusion_transformers_amd import synth
    cfg = synth.CONFIGS["mixed"]
    shape = R.shape_of(cfg)
    _, r32 = synth.rotation_matrices(cfg.split)
    rr = R.RopeRotDevice(shape, r32)
    mask = synth.fallback_mask(cfg)
    ws = torch.empty(R.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    o = torch.empty((cfg.B, cfg.H, cfg.N, cfg.D), dtype=torch.float16, device="cuda")
    prep = R.PreparedDevice(shape, with_rope=True)
    n_fb = int(mask.sum())
    n_i4 = cfg.BH - n_fb
    per_step = []
    for s in range(steps):
        q, k, v = synth.all_heads_qkv(cfg, s)
        qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
        del q, k, v
        ms = time_calls(lambda: R.mixed_fwd(shape, qd, kd, vd, rr, mask, ws, o), 1)
        # the two attention kernels of the step on their own
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, mask)
        i4 = time_calls(lambda: R.int4_fwd(shape, prep, o, mask=mask), 1)
        f16 = time_calls(lambda: R.fp16_fwd_prepared(shape, prep, o, head_select=mask), 1)
        per_step.append({"step": s, "ms": round(ms, 4), "int4_attn_ms": round(i4, 4),
                         "fp16_attn_ms": round(f16, 4)})
        del qd, kd, vd
    ms = float(np.mean([p["ms"] for p in per_step]))
    i4 = float(np.mean([p["int4_attn_ms"] for p in per_step]))
    f16 = float(np.mean([p["fp16_attn_ms"] for p in per_step]))
    unit = 4.0 * cfg.N ** 2 * cfg.D
    ops = unit * cfg.BH
    print(f"[bench] mixed {steps} step(s): " +
          ", ".join(f"step {p['step']} {p['ms']:.3f} ms" for p in per_step), file=sys.stderr,
          flush=True)
    del prep, ws, o
    torch.cuda.empty_cache()
    return {"workload": f"mixed: 720p shape (B=1 H=40 N=75600 D=128), {n_fb} of 40 heads FP16 "
                        f"(seeded mask, fixed across steps), fresh seeded Q/K/V per step, one "
                        f"rotattn_mixed_fwd per step",
            "steps": steps, "fp16_heads": n_fb, "per_step": per_step,
            "ms_per_step": round(ms, 4), "effective_tops": round(ops / (ms * 1e-3) / 1e12, 2),
            "int4_attn_ms": round(i4, 4),
            "int4_attn_i8_peak_frac": round(unit * n_i4 / (i4 * 1e-3) / 1e12 / PEAK_I8_TOPS, 4),
            "fp16_attn_ms": round(f16, 4),
            "fp16_attn_f16_peak_frac": round(unit * n_fb / (f16 * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}


def bench_workload(name: str, reps: int = 5):
    """Side figure: one step (prologue + INT4 attention, every head INT4) of
    another workload, inputs resident in HBM."""
    import torch
    from video_diffusion_transformers_amd import rotattn as R
    from video_diffusion_transformers_amd import synth
    cfg = synth.CONFIGS[name]
    shape = R.shape_of(cfg)
    q, k, v = synth.all_heads_qkv(cfg, 0)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    del q, k, v
    _, r32 = synth.rotation_matrices(cfg.split)
    rr = R.RopeRotDevice(shape, r32)
    prep = R.PreparedDevice(shape, with_rope=False)
    o = torch.empty((cfg.B, cfg.H, cfg.N, cfg.D), dtype=torch.float16, device="cuda")

    def step():
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, None)
        R.int4_fwd(shape, prep, o)

    step_ms = time_calls(step, reps)
    pro_ms = time_calls(lambda: R.prepare_qkv(shape, qd, kd, vd, rr, prep, None), reps)
    i4_ms = time_calls(lambda: R.int4_fwd(shape, prep, o), reps)
    ops = 4.0 * cfg.BH * cfg.N ** 2 * cfg.D
    pro_alg, _ = prologue_bytes(cfg.BH, cfg.N, cfg.D)
    del qd, kd, vd, prep, o
    torch.cuda.empty_cache()
    print(f"[bench] {name}: step {step_ms:.3f} ms (prologue {pro_ms:.3f}, int4 {i4_ms:.3f})",
          file=sys.stderr, flush=True)
    return {"workload": f"{name}: B={cfg.B} H={cfg.H} grid {'x'.join(map(str, cfg.grid))} "
                        f"N={cfg.N} D={cfg.D}, every head INT4",
            "ms_per_step": round(step_ms, 4), "effective_tops": round(ops / (step_ms * 1e-3) / 1e12, 2),
            "int4_attn_ms": round(i4_ms, 4),
            "int4_attn_i8_peak_frac": round(ops / (i4_ms * 1e-3) / 1e12 / PEAK_I8_TOPS, 4),
            "prologue_ms": round(pro_ms, 4),
            "prologue_hbm_frac": round(pro_alg / (pro_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def cpu_baseline(cfg, ops, heads: int | None = None, rows: int = 256):
    """The CPU oracle on this host's cores: for `heads` heads of the workload
    (default: one per core, at most 16), the prologue over all N tokens plus
    the INT4 attention of `rows` sampled query rows each, one head per worker
    process (the oracle is single threaded per head).  The measured wall time is scaled by the ratio of the
    whole workload's work (every head, every query row) to the sample's, both
    from the workers' own per-head timings."""
    from oracle import parallel
    from video_diffusion_transformers_amd import synth
    visible = parallel.host_cores()
    if heads is None:
        heads = min(visible, parallel.MAX_WORKERS, cfg.BH)   # one head per core
    workers = min(visible, parallel.MAX_WORKERS, heads)
    bhs = [int(x) for x in np.linspace(0, cfg.BH - 1, heads).round()]
    jobs = [(bh, synth.sampled_rows(cfg, bh, rows), False) for bh in bhs]
    t0 = time.perf_counter()
    _, secs = parallel.run_heads(cfg, 0, jobs, workers=workers)
    wall = time.perf_counter() - t0
    pro = np.array([secs[bh][0] for bh in bhs])
    att = np.array([secs[bh][1] for bh in bhs])
    sample_work = float(np.sum(pro + att))
    full_work = cfg.BH * (float(pro.mean()) + float(att.mean()) * cfg.N / rows)
    full_wall = wall * full_work / sample_work
    print(f"[bench] cpu oracle: {heads} heads x ({cfg.N}-token prologue + {rows} query rows) on "
          f"{workers} workers in {wall:.1f} s -> {full_wall / 3600:.1f} h extrapolated",
          file=sys.stderr, flush=True)
    return {"value": round(ops / full_wall / 1e12, 6), "unit": "TOP/s", "cores": int(workers),
            "host_cores_visible": int(visible), "kind": "oracle",
            "sample": f"{heads} heads of {cfg.name} (heads {bhs}), each: prologue over all {cfg.N} "
                      f"tokens ({pro.mean():.2f} s) + INT4 attention of {rows} seeded query rows "
                      f"({att.mean():.2f} s), one head per process on {workers} cores: "
                      f"{wall:.1f} s wall; extrapolated to {cfg.BH} heads x {cfg.N} rows by the "
                      f"measured per-head work = {full_wall:.0f} s",
            "measured_s": round(wall, 2), "extrapolated": True}


if __name__ == "__main__":
    main()

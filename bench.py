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
of the dominant kernel (the INT4 attention, timed with HIP events on the
stream it runs on, with the VALU-busy share of the unit that bounds it), the
per-kernel times, and the CPU oracle timed on a bounded
sample on this host (cpu_baseline).
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
PEAK_I8_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POPS)
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA (2.5 PFLOPS)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (8 TB/s)
PMC_FILE = os.path.join(ROOT, "profiles", "int4_attn_f8_720p_pmc.txt")
SQ_FILE = os.path.join(ROOT, "profiles", "int4_attn_f8_720p_sq_counters.txt")
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
    ap.add_argument("--mixed-steps", type=int, default=2,
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
    prep = R.PreparedDevice(shape, with_rope=True)
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
            R.fp16_fwd(shape, prep, o, head_select=mask)
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
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_I8_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_I8_TOPS, 4), "traffic": traffic,
                "kernel": "k_int4_attn_f8<128>", "algorithmic_ops_per_launch": int4_ops,
                "limiter": "valu", "limiter_busy": valu_busy_from_profile(args.workload)}
    # prologue: algorithmic HBM bytes per token per head (read Q,K,V fp16; write
    # Q,K,V codes one byte each in the FP8-lane layout; block scales are negligible)
    k1_bytes = BH * N * (3 * 2 * D + 3 * D)
    kernels = {
        "prologue_ms": round(float(k1.mean()), 4),
        "prologue_hbm_frac": round(k1_bytes / (float(k1.mean()) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "int4_attn_ms": round(k2_ms, 4),
        "int4_attn_ms_min": round(float(k2.min()), 4),
        "int4_attn_i8_peak_frac": round(achieved / PEAK_I8_TOPS, 4),
        "fp16_attn_ms": round(float(k3.mean()), 4),
        "event_step_ms": round(float(tot.mean()), 4),
    }

    if not args.no_extras:
        # the same INT4 attention on the nibble-packed layout (i8 MFMA kernel)
        # (fallback heads, if any, need the fp16 RoPE'd buffers as well)
        prep_p = R.PreparedDevice(shape, with_rope=n_fb > 0, layout=R.LAYOUT_PACKED)
        R.prepare_qkv(shape, qd, kd, vd, rr, prep_p, mask)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        R.int4_fwd(shape, prep_p, o, mask=mask)
        e0.record()
        for _ in range(3):
            R.int4_fwd(shape, prep_p, o, mask=mask)
        e1.record()
        torch.cuda.synchronize()
        kernels["int4_attn_packed_i8_ms"] = round(e0.elapsed_time(e1) / 3, 4)
        del prep_p

        # mixed_fwd (one C call) on the same inputs, as a cross-check of the sequence
        ws = torch.empty(R.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        R.mixed_fwd(shape, qd, kd, vd, rr, mask, ws, o)
        e0.record()
        for _ in range(3):
            R.mixed_fwd(shape, qd, kd, vd, rr, mask, ws, o)
        e1.record()
        torch.cuda.synchronize()
        kernels["mixed_fwd_call_ms"] = round(e0.elapsed_time(e1) / 3, 4)
        del ws

        # INT4 output of every head, kept for the per-head error report below
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, None)
        R.int4_fwd(shape, prep, o, mask=None)
        o_int4 = o.clone()

        # FP16 FlashAttention on every head of the same shape (kernel-level analogue
        # of the full-precision baseline) -- context figure
        all_fb = np.ones(BH, np.uint8)
        R.prepare_qkv(shape, qd, kd, vd, rr, prep, all_fb)
        e0.record()
        R.fp16_fwd(shape, prep, o, head_select=all_fb)
        e1.record()
        torch.cuda.synchronize()
        R.fp16_fwd(shape, prep, o, head_select=all_fb)
        e2 = torch.cuda.Event(enable_timing=True)
        e2.record()
        torch.cuda.synchronize()
        f16_ms = e1.elapsed_time(e2)
        kernels["fp16_attn_all_heads_ms"] = round(f16_ms, 4)
        kernels["fp16_attn_f16_peak_frac"] = round(ops / (f16_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)
        kernels["int4_vs_fp16_kernel_speedup"] = round(f16_ms / k2_ms, 3) if n_int4 == BH else None
        print(f"[bench] fp16 all heads {f16_ms:.3f} ms", file=sys.stderr, flush=True)
        from video_diffusion_transformers_amd import fallback
        kernels["int4_vs_fp16_head_error"] = dict(
            reference="FP16 attention kernel, same inputs",
            **fallback.report(fallback.head_rel_error(o_int4, o)))

        # the rotation merged into RoPE (seeded pair phases in the tables, no
        # dense rotation): prologue time and the same error report
        rr_m = R.RopeRotDevice(shape, None, phases=synth.mergeable_phases(cfg.split))
        R.prepare_qkv(shape, qd, kd, vd, rr_m, prep, None)
        e0.record()
        for _ in range(3):
            R.prepare_qkv(shape, qd, kd, vd, rr_m, prep, None)
        e1.record()
        torch.cuda.synchronize()
        kernels["prologue_merged_rotation_ms"] = round(e0.elapsed_time(e1) / 3, 4)
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

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, q, k, v, r32, ops)

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
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} H={H} grid {'x'.join(map(str, cfg.grid))} "
                               f"N={N} D={D} split {'/'.join(map(str, cfg.split))}, "
                               f"{BH - n_fb} INT4 heads + {n_fb} FP16 heads, seeded synthetic "
                               f"fp16 Q/K/V (RoPE-partition outlier channels, sparse V token "
                               f"outliers)",
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": D,
                   "parallelism": "single GPU"},
        "percent_i8_peak_step": round(100 * value / PEAK_I8_TOPS, 2),
        "roofline": roofline,
        "kernels": kernels,
        "mixed": mixed,
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
    copies around the attention, and against FP16 attention on every head."""
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
    res["int4_vs_fp16_block_speedup"] = round(res["fp16_fused_ms"] / res["int4_fused_ms"], 3)
    print(f"[bench] DiT block: {res}", file=sys.stderr, flush=True)
    del blk, x
    torch.cuda.empty_cache()
    return dict(workload=f"720p shape, width {width}, QKV projection + attention + output "
                         f"projection, random weights (timing only)", **res)


def bench_mixed(steps: int):
    """The mixed workload: 720p shape, one rotattn_mixed_fwd per denoising step
    with fresh inputs and a per-step fallback mask (step 0: every head FP16;
    later steps: a seeded quarter of the heads FP16).  Side figure."""
    import torch
    from video_diffusion_transformers_amd import rotattn as R
    from video_diffusion_transformers_amd import synth
    cfg = synth.CONFIGS["mixed"]
    shape = R.shape_of(cfg)
    _, r32 = synth.rotation_matrices(cfg.split)
    rr = R.RopeRotDevice(shape, r32)
    sched = synth.fallback_schedule(cfg, steps, early_fp16_steps=1)[:, 0]
    ws = torch.empty(R.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    o = torch.empty((cfg.B, cfg.H, cfg.N, cfg.D), dtype=torch.float16, device="cuda")
    per_step = []
    for s in range(steps):
        q, k, v = synth.all_heads_qkv(cfg, s)
        qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
        R.mixed_fwd(shape, qd, kd, vd, rr, sched[s], ws, o)      # warm
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        R.mixed_fwd(shape, qd, kd, vd, rr, sched[s], ws, o)
        e1.record()
        torch.cuda.synchronize()
        per_step.append({"step": s, "fp16_heads": int(sched[s].sum()),
                         "ms": round(e0.elapsed_time(e1), 4)})
        del qd, kd, vd
    ms = float(np.mean([p["ms"] for p in per_step]))
    ops = 4.0 * cfg.B * cfg.H * cfg.N ** 2 * cfg.D
    print(f"[bench] mixed {steps} step(s): " +
          ", ".join(f"step {p['step']} ({p['fp16_heads']} FP16 heads) {p['ms']:.3f} ms"
                    for p in per_step), file=sys.stderr, flush=True)
    return {"workload": "720p shape, per-step fallback mask (step 0 all heads FP16, then 10 of "
                        "40 heads FP16, seeded), fresh inputs per step",
            "steps": steps, "per_step": per_step, "ms_per_step": round(ms, 4),
            "effective_tops": round(ops / (ms * 1e-3) / 1e12, 2)}


def cpu_baseline(cfg, q, k, v, r32, ops):
    """The CPU oracle on this host: prologue of one head over all tokens plus
    INT4 attention of a few query rows of that head, extrapolated to the whole
    workload in the metric's unit."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    rows_n = 48
    t0 = time.perf_counter()
    tabs = O.all_rope_tables(cfg.grid, cfg.split)
    t_tab = time.perf_counter() - t0
    qh, kh, vh = q[0, 0], k[0, 0], v[0, 0]
    t0 = time.perf_counter()
    prep = O.prepare_head(qh, kh, vh, tabs, r32, cfg.grid, cfg.split)
    t_pro = time.perf_counter() - t0
    rows = np.arange(rows_n) * (cfg.N // rows_n)
    t0 = time.perf_counter()
    O.int4_attention(prep["q_codes"], prep["q_scale_l2"], prep["k_codes"], prep["k_scale"],
                     prep["v_codes"], prep["v_scale"], rows)
    t_att = time.perf_counter() - t0
    full_s = t_tab + cfg.BH * t_pro + cfg.BH * t_att * cfg.N / rows_n
    print(f"[bench] cpu oracle: prologue {t_pro:.2f}s/head, attention {t_att:.2f}s/{rows_n} rows "
          f"-> {full_s / 3600:.1f} h extrapolated", file=sys.stderr, flush=True)
    return {"value": round(ops / full_s / 1e12, 6), "unit": "TOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"head 0 of {cfg.name}: prologue over all {cfg.N} tokens ({t_pro:.2f} s) + "
                      f"INT4 attention of {rows_n} query rows ({t_att:.2f} s), extrapolated to "
                      f"{cfg.BH} heads x {cfg.N} rows = {full_s:.0f} s",
            "measured_s": round(t_tab + t_pro + t_att, 2)}


if __name__ == "__main__":
    main()

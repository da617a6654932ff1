"""Builds librotattn.so in-tree with hipcc for gfx950 (no GPU needed).

    python -m video_diffusion_transformers_amd.build_lib [--jobs N]

Every HIP source is compiled for gfx950 only, with FP contraction off (the
prologue's rounding is part of the bit-exact contract; wanted FMAs are written
as fmaf) and packed-FP32 code generation disabled.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librotattn.so")
MICROBENCH = os.path.join(HERE, "rotattn_microbench")
SOURCES = ["rotattn_host.cpp", "prologue.hip", "int4_attn.hip", "fp16_attn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    # the microbenchmark executable (roofline denominators, copy calibration)
    r = subprocess.run([HIPCC, *FLAGS, "-x", "hip", os.path.join(CSRC, "microbench.hip"),
                        "-o", MICROBENCH + ".tmp"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("microbench build failed:\n" + r.stdout + r.stderr)
    os.replace(MICROBENCH + ".tmp", MICROBENCH)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    print(build(ap.parse_args().jobs))

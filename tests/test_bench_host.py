"""Host logic of bench.py (no GPU): the roofline's traffic and VALU-share
fields come from the committed rocprofv3 summaries only for the workload they
were taken on and only while the INT4 kernel source still has the hash the
summaries record; otherwise both are null."""
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_profiles_match_current_kernel_source():
    # the committed summaries were taken on the committed kernel
    assert bench.traffic_from_profile(bench.PROFILED_WORKLOAD) is not None
    busy = bench.valu_busy_from_profile(bench.PROFILED_WORKLOAD)
    assert busy is not None and 0.0 < busy <= 1.0


@pytest.mark.parametrize("workload", ["480p", "small", "mixed"])
def test_other_workloads_report_null(workload):
    assert bench.traffic_from_profile(workload) is None
    assert bench.valu_busy_from_profile(workload) is None


def test_stale_profiles_report_null(tmp_path, monkeypatch):
    # a kernel source that differs from the one the summaries were taken on
    src = tmp_path / "int4_attn.hip"
    shutil.copyfile(bench.KERNEL_SRC, src)
    with open(src, "a") as f:
        f.write("\n// edited\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    assert bench.traffic_from_profile(bench.PROFILED_WORKLOAD) is None
    assert bench.valu_busy_from_profile(bench.PROFILED_WORKLOAD) is None


def test_traffic_is_scaled_counter_bytes():
    # hbm_bytes_per_launch = (FETCH_SIZE * fetch factor + WRITE_SIZE * write factor) * 1024
    vals = {}
    with open(bench.PMC_FILE) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    fetch = float(vals["fetch_size_kib_per_dispatch"])
    write = float(vals["write_size_kib_per_dispatch"])
    ff = float(vals["fetch_calibration_factor"])
    wf = float(vals.get("write_calibration_factor", "1.0"))
    expect = (fetch * ff + write * wf) * 1024
    assert abs(bench.traffic_from_profile(bench.PROFILED_WORKLOAD) - expect) <= 1e-6 * expect

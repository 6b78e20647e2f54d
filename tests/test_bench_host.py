"""Host-side checks of the benchmark script (no GPU).

* The one-GPU contract: more than one GPU is refused before anything
  touches a device.
* The committed profile summaries reproduce the roofline figures the bench
  line reports: every derived number in them is recomputed here from the
  raw ones, and the algorithmic bytes from the W4 format itself (packed
  codes, fp32 scales and packed zero points per weight, plus x and y), so
  a summary whose figures do not follow from its own measurements, or a
  bench that counts bytes differently from the format, fails.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _fields(name):
    b = _bench()
    f = b.read_summary_fields(os.path.join(ROOT, b.PROFILE_DIR, name))
    assert f, f"no key: value lines in {name}"
    return f


def _close(a, b, rel=2e-3):
    return abs(a - b) <= rel * max(abs(a), abs(b))


def _matmul_bytes(K, N):
    # codes K*N/2, scales (K/32)*N fp32, zero points (K/32)*N/2, x 4K, y 4N (M = 1)
    return K * N // 2 + (K // 32) * N * 4 + (K // 32) * N // 2 + 4 * K + 4 * N


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_pass_bytes_follow_from_the_format():
    shapes = synth.DENSE38_SHAPES
    assert len(shapes) == 4
    per_layer = sum(_matmul_bytes(K, N) for K, N in shapes)
    assert 32 * per_layer == 2_327_838_720
    # the per-launch average the roofline divides by
    assert 32 * per_layer // 128 == 18_186_240
    f = _fields(_bench().TRAFFIC_SUMMARY)
    assert int(f["algorithmic_bytes_per_launch"]) == 32 * per_layer // 128


def test_trace_summary_reproduces_the_bench_roofline():
    b = _bench()
    f = _fields(b.TRACE_SUMMARY)
    pass_bytes = 32 * sum(_matmul_bytes(K, N) for K, N in synth.DENSE38_SHAPES)
    ms = float(f["bench_ms_per_step"])
    untraced_us = float(f["gemv_avg_us_bench_untraced"])
    traced_us = float(f["gemv_avg_us_bench_traced_run"])
    rocprof_us = float(f["gemv_avg_us_rocprof"])
    assert int(f["gemv_dispatches"]) % 128 == 0
    # value: the pass's bytes over the time per pass
    assert _close(float(f["bench_value_GB_s"]), pass_bytes / (ms * 1e-3) / 1e9)
    # every one of the 128 launches is the GEMV: the untraced launch average
    # is the pass time over 128, and the kernels fit inside the step
    assert _close(untraced_us, 1e3 * ms / 128)
    assert 128 * untraced_us <= 1e3 * ms * (1 + 2e-3)
    achieved = float(f["roofline_achieved_GB_s"])
    assert _close(achieved, pass_bytes / 128 / (untraced_us * 1e-6) / 1e9)
    assert _close(float(f["roofline_frac"]), achieved / HBM_PEAK_GBS)
    assert _close(float(f["tracer_overhead"]), traced_us / untraced_us)
    # the tracer only slows the kernels down: the traced kernel durations are
    # not below the untraced launch average
    assert rocprof_us >= untraced_us * (1 - 2e-3)
    assert traced_us >= untraced_us


def test_traffic_summary_reproduces_its_calibration():
    f = _fields(_bench().TRAFFIC_SUMMARY)
    wf = float(f["write_factor"])
    ff = float(f["fetch_factor"])
    # the copy kernel reads the bytes it writes: the fetch factor is what
    # FETCH_SIZE reads for them over what WRITE_SIZE (scaled) reads
    copy_true_kib = float(f["write_copy_kib"]) / wf
    assert _close(ff, float(f["fetch_copy_kib"]) / copy_true_kib)
    fetch = float(f["fetch_bytes_per_launch"])
    write = float(f["write_bytes_per_launch"])
    assert _close(fetch, float(f["fetch_kib_per_launch_raw"]) * 1024 / ff)
    assert _close(write, float(f["write_kib_per_launch_raw"]) * 1024 / wf, rel=2e-2)
    alg = float(f["algorithmic_bytes_per_launch"])
    assert _close(float(f["traffic_over_algorithmic"]), (fetch + write) / alg)
    # no kernel can read less than its codes, scales and zero points
    assert fetch + write >= 0.99 * alg
    # an independent counter: read requests to DRAM, scaled by the same copy,
    # agree with FETCH_SIZE within 10%
    assert _close(float(f["rdreq_gemv_bytes_scaled_by_copy"]), fetch, rel=0.10)


@pytest.mark.parametrize("name", ["k_gemv_kmajor_dense38_m1_kernel_trace.md",
                                  "k_gemv_kmajor_dense38_m1_traffic.md"])
def test_summaries_name_their_command(name):
    with open(os.path.join(ROOT, "profiles", name)) as fh:
        text = fh.read()
    assert "rocprofv3" in text and "bench.py" in text

"""bench.py's command line on the host: a request for more than one GPU is
refused with a message before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_reports_host_and_single_core():
    """The CPU baseline of the 256 x 512 fp32 bucket (the fp64 oracle on the
    host, milliseconds of work): a rate on the BLAS pool, the same sample on one
    core, and the host's CPU description."""
    import types
    sys.path.insert(0, ROOT)
    import bench
    from matrix_optimizers_amd import workloads as wlmod
    out = bench.cpu_baseline(wlmod.get("single_256x512_f32"), types.SimpleNamespace())
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["single_core"]["cores"] == 1 and out["single_core"]["value"] > 0
    assert out["host"]["usable_cpus"] >= 1
    big = bench.SINGLE_CORE_WORKLOADS
    assert "large_single" not in big   # the default bucket's sample stays bounded to the all-core run

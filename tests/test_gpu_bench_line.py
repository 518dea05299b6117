"""bench.py end to end on the GPU: one short run of the tiny workload prints
one JSON line with the fields its consumers read (metric, value, roofline,
cpu_baseline, workspace_errors), and the figures in it are consistent; the
chunked fp8 workload on two streams does too, and so do the back-to-back
and copy-calibration modes."""

import json
import os
import subprocess
import sys

import pytest

from tests.gpu_helpers import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_consistent_json_line():
    print("case: bench.py --workload tiny --steps 3 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1", "--cpu-tokens", "64"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "workspace_errors"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["workspace_errors"] == 0
    assert d["config"]["workload"] == "tiny"
    # value is the algorithmic bytes over the step time
    assert abs(d["value"] - d["alg_bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9) \
        <= 0.01 * d["value"] + 0.01
    rf = d["roofline"]
    assert rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0


def test_bench_chunked_fp8_on_two_streams():
    """The chunked fp8 workload with the configuration's two-stream schedule
    (--streams 2): one JSON line, its config naming two streams and four
    chunks, and no bounded wait that gave up."""
    print("case: bench.py --workload fp8_t32768 --streams 2 --steps 2 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "fp8_t32768", "--streams", "2", "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["config"]["workload"] == "fp8_t32768"
    assert d["config"]["streams"] == 2 and d["config"]["chunks"] == 4
    assert d["workspace_errors"] == 0
    assert d["value"] > 0 and d["roofline"]["frac"] > 0
    assert abs(d["value"] - d["alg_bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9) \
        <= 0.01 * d["value"] + 0.01


def _one_line(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_bench_back_to_back_and_copy_calibration():
    """--back-to-back times uninterrupted steps with the Infinity Cache left
    warm, and says so in its line; --copy-calibration (the reference copy the
    rocprofv3 byte counters are scaled by) reports the bytes it moves."""
    print("case: bench.py --workload tiny --back-to-back; --copy-calibration", flush=True)
    d = _one_line(["--workload", "tiny", "--steps", "3", "--warmup", "1", "--back-to-back",
                   "--no-cpu-baseline"])
    assert d["config"]["mall_flush_between_steps"] is False
    assert d["value"] > 0 and d["workspace_errors"] == 0
    c = _one_line(["--copy-calibration"])
    assert c["copy_calibration_bytes_read"] == c["copy_calibration_bytes_written"] > 0

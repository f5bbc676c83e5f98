"""bench.py's output contract: one JSON line with the decode metric, its
roofline and the CPU oracle beside it (a short run on the GPU), and the
refusal of more than one GPU (on the CPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.gpu
def test_bench_line_contract():
    """A short decode run (3 timed steps) prints one JSON line whose fields
    agree with each other: throughput = bytes per step / step time, the
    roofline fraction = achieved / peak, tokens per second = batch / step."""
    print("[gpu] bench.py short run", flush=True)
    r = _bench("--steps", "3", "--warmup", "2", "--cpu-seconds", "1", "--no-next", "--cold", "1", "--in-step", "1",
               "--burst", "2")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    a = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in a, key
    assert a["n_gpus"] == 1 and a["steps"] == 3 and a["warmup"] == 2
    assert a["higher_is_better"] is True and a["vs_baseline"] is None
    assert a["dtype"] == "bf16" and a["config"]["workload"] == "c2_gqa_bf16"
    assert a["value"] > 0 and a["ms_per_step"] > 0
    # value is K/V GB/s of the whole step: bytes per step over the step time
    step_bytes = a["value"] * 1e9 * a["ms_per_step"] * 1e-3
    assert 4e8 < step_bytes < 7e8, step_bytes
    if "tokens_per_s" in a:
        assert abs(a["tokens_per_s"] * a["ms_per_step"] * 1e-3 - 64) < 0.5
    rf = a["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # the pass alone runs no slower than the whole step it sits in
    assert rf["achieved"] >= a["value"] * 0.98
    cb = a["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1

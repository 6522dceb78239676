"""The benchmark's JSON line on the GPU: the fields a reader of the line relies on, and their
consistency (value against the dense-equivalent FLOPs, the roofline fraction, one duration per
timed step). A short run: 3 timed steps after 2 warm-up steps, no secondary workload, a 1 s CPU
oracle sample."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def test_bench_line_fields_and_consistency():
    steps, warmup = 3, 2
    print(f"bench.py --steps {steps} --warmup {warmup} (480p)", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", str(steps), "--warmup",
                        str(warmup), "--secondary", "", "--cpu-seconds", "1"], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    line = json.loads(p.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == steps and line["warmup"] == warmup
    assert line["higher_is_better"] is True and line["dtype"] == "bf16"
    assert line["config"]["workload"] == "480p" and line["config"]["tokens"] == 37632
    # value = 4*B*H*N^2*d per layer over the time per layer
    dense = 4.0 * 1 * 12 * 37632 ** 2 * 128
    assert line["value"] == pytest.approx(dense / (line["ms_per_step"] * 1e-3) / 1e12, rel=1e-3)
    rf = line["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert 0.0 < rf["frac"] < 1.0
    cb = line["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    ts = line["timed_steps_ms"]
    assert len(ts) == steps and all(t > 0 for t in ts)
    # the per-step durations tile the timed region (up to the events around it)
    assert sum(ts) / steps == pytest.approx(line["ms_per_step"], rel=0.1)
    print(f"value {line['value']:.1f} TFLOP/s, {line['ms_per_step']} ms per layer, steps {ts}", flush=True)

"""bench.py's host-side pieces: the one-GPU guard and the order statistics it reports."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in json.loads(p.stdout.strip().splitlines()[-1])["error"]


def test_median():
    assert bench.median([3.0]) == 3.0
    assert bench.median([4.0, 1.0, 3.0]) == 3.0
    assert bench.median([4.0, 1.0, 3.0, 2.0]) == 2.5


def test_evicts_twice_the_last_level_cache():
    assert bench.EVICT_BYTES == 2 * 256 * (1 << 20)

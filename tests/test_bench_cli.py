"""bench.py's command line on the CPU: it measures one GPU and refuses any other count before touching one."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT, env=env)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _bench(env=dict(os.environ, WORLD_SIZE="2"))
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""

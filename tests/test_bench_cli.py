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


def test_shader_clocks_parsed_from_amd_smi_json():
    """The clock sampler reads gfx_N clocks per GPU from amd-smi's JSON, in die order, and ignores the rest."""
    sys.path.insert(0, ROOT)
    import bench

    die = lambda mhz: {"clk": {"value": mhz, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"}}
    data = {"gpu_data": [{"gpu": 0, "clock": {"gfx_1": die(1800), "gfx_0": die(1700), "gfx_10": die(1900),
                                                "mem_0": die(1300), "gfx_2": {"clk": "N/A"}}},
                         {"gpu": 3, "clock": {"gfx_0": die(95)}}]}
    assert bench.gfx_clocks_from_amd_smi(data) == {0: [1700.0, 1800.0, 1900.0], 3: [95.0]}
    assert bench.gfx_clocks_from_amd_smi(data["gpu_data"]) == {0: [1700.0, 1800.0, 1900.0], 3: [95.0]}
    assert bench.gfx_clocks_from_amd_smi({"gpu_data": [{"gpu": 0, "clock": {}}]}) is None
    assert bench.gfx_clocks_from_amd_smi("not json") is None

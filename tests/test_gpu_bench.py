"""bench.py end to end on the GPU, on the tiny workload: the JSON line it prints
keeps its contract, and the per-configuration records report bit-exact outputs."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_bench(*args):
    print(f"[gpu-case] bench.py {' '.join(args)}", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    return [json.loads(line) for line in res.stdout.splitlines() if line.startswith("{")]


def test_bench_line_contract():
    (line,) = run_bench("--workload", "tiny", "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
                        "--no-per-config")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 1
    assert line["value"] > 0 and line["config"]["workload"] == "tiny"
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3


def test_records_are_bit_exact():
    recs = run_bench("--records", "--records-workload", "tiny", "--steps", "5")
    assert [(r["mode"], r["chunked"]) for r in recs] == [(0, False), (1, False)]
    for r in recs:
        assert r["bit_exact"] is True and r["launches_timed"] == 5
        assert r["ncores"] == 2 and r["oracle_ncore_s"] is not None    # tiny: w = 2 senders
        assert r["t_min_us"] <= r["t_median_us"] and len(r["input_sha256"]) == 64


def test_per_config_covers_the_five_workloads():
    """The default line's per_config: every workload in both modes (and the
    four-plane one chunked), each bit-exact against the oracle."""
    (line,) = run_bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    pc = line["per_config"]
    assert sorted(pc) == sorted(["tiny", "mid", "video_dit", "chunked", "chunked_chunked", "awkward"])
    for name, entry in pc.items():
        for m in ("mode0", "mode1"):
            assert entry[m]["bit_exact"] is True, (name, m)
            assert entry[m]["us"] > 0 and 0 <= entry[m]["frac"] < 1, (name, m)
    assert pc["chunked_chunked"]["mode0"]["launches"] == 1

"""bench.py end to end on the GPU: a short default run (every sub-measurement on) prints
one JSON line with the fields the measurement needs."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_bench_line_with_every_sub_measurement():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench.py --steps 3 --warmup 1 --replicas 1 --cpu-seconds 1", flush=True)
    r = subprocess.run([sys.executable, "-u", "bench.py", "--steps", "3", "--warmup", "1", "--replicas", "1",
                        "--cpu-seconds", "1"], cwd=ROOT, capture_output=True, text=True, timeout=850)
    assert r.returncode == 0, r.stderr[-4000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "ms_per_step", "roofline", "cpu_baseline", "cpu_baseline_1_thread",
                "graph_replay", "prefill", "fp8_kv", "schedule_61", "cache_append", "fp4_indexer", "kernels"):
        assert key in line, key
    assert line["value"] > 0 and line["n_gpus"] == 1
    assert line["graph_replay"]["outputs_equal_eager"]
    rf = line["roofline"]
    assert rf["bound"] == "hbm" and 0 < rf["frac"] < 1 and rf["peak"] == 8000.0

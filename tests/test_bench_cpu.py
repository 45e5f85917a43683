"""bench.py host logic without a GPU: the single-GPU contract and the layer schedule."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_layer_schedule_of_the_61_layer_stack():
    s = bench.SCHEDULE
    assert len(s) == 62 and s[-1] == "swa"                       # 61 layers + the MTP block
    assert s[0] == s[1] == "hca" and s[2] == "csa" and s[3] == "hca" and s[60] == "csa"
    assert all(s[i] != s[i + 1] for i in range(2, 60))           # alternating from layer 2 to 60
    assert (s.count("csa"), s.count("hca"), s.count("swa")) == (30, 31, 1)


def test_kv_bytes_per_token():
    kvb = bench.kv_bytes_per_token()
    # CSA: a 2 KB bf16 K|V entry and a 68-byte MXFP4 key per 4 tokens; HCA: 2 KB per 128 tokens
    assert kvb["csa"] == (2048 + 68) / 4 and kvb["hca"] == 2048 / 128 and kvb["swa"] == 0

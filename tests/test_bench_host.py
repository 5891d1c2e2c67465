"""bench.py's host-side contract, without a GPU: it refuses more than one GPU before touching one,
reports counter-measured HBM traffic only while the kernel sources still hash to the value recorded
with the counters, and prices the roofline against the published peaks."""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""       # no JSON line


def committed_traffic():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("workload", sorted(committed_traffic()))
def test_traffic_is_reported_while_the_sources_match(workload):
    tj = committed_traffic()
    (part, ent), = tj[workload].items()
    args = types.SimpleNamespace(traffic_json=os.path.join(ROOT, "profiles", "traffic.json"))
    assert bench.traffic_for(args, workload, part) == ent["bytes_per_launch"]
    assert bench.traffic_for(args, workload, "no such part") is None


def test_traffic_turns_null_when_the_sources_change(tmp_path):
    tj = committed_traffic()
    stale = tmp_path / "traffic.json"
    for ent in tj["block"].values():
        ent["source_sha256_prefix"] = "0" * 16          # counters taken on other sources
    stale.write_text(json.dumps(tj))
    args = types.SimpleNamespace(traffic_json=str(stale))
    assert bench.traffic_for(args, "block", "dca") is None
    assert bench.traffic_for(types.SimpleNamespace(traffic_json=str(tmp_path / "missing.json")), "block", "dca") is None


def test_roofline_prices_against_the_published_peaks():
    per = {"dca": {"tflops": 1250.0, "ms_avg": 28.0}, "fm": {"gbs_algorithmic": 4000.0, "ms_avg": 0.5}}
    r = bench.roofline_of("block", "dca", per, {"dca": 3.5e13}, {"dca": 8.6e9}, 123)
    assert (r["bound"], r["unit"], r["peak"], r["frac"], r["traffic"]) == ("mfma", "TFLOP/s", 2500.0, 0.5, 123)
    r = bench.roofline_of("fm", "fm", per, {"fm": 1e11}, {"fm": 2.15e9}, None)
    assert (r["bound"], r["unit"], r["peak"], r["frac"], r["traffic"]) == ("hbm", "GB/s", 8000.0, 0.5, None)

"""Host-side logic of bench.py (no GPU): the one-GPU guard, the workload
records it prints, and the rule that measured traffic is reported only for
the library the counters were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from qsa_inputs import ALL_CONFIGS, PoolConfig  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


@pytest.mark.parametrize("cfg", ALL_CONFIGS, ids=[c.name for c in ALL_CONFIGS])
def test_workload_records_are_complete(cfg):
    rec = bench.workload_config(cfg)
    json.dumps(rec)
    assert rec["workload"] == cfg.name
    assert rec["valid_slots"] == cfg.valid_slots() > 0
    assert rec["head_dim"] == 256 and rec["Hq"] % rec["Hkv"] == 0
    if isinstance(cfg, PoolConfig):
        assert rec["n_slots"] == cfg.n_slots and len(rec["requests"]) == len(cfg.requests)
        assert sum(r["new"] for r in rec["requests"]) == rec["T"]
    else:
        assert rec["T_kv"] >= rec["q_pos0"] + rec["T"]


def test_traffic_only_for_the_profiled_library(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_sha": "abc", "fetch_bytes_per_launch": 1000.4, "write_bytes_per_launch": 20.2}
    (prof / "qsa_prefill_kernel_w_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", "abc") == 1021
    assert bench.measured_traffic("w", "abd") is None
    assert bench.measured_traffic("other", "abc") is None


def test_committed_profiles_name_their_library():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.endswith("_traffic.json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", name)))
            assert len(rec["kernel_sha"]) == 16 and rec["fetch_bytes_per_launch"] > 0
            assert all("bench.py" in c for c in rec["commands"])

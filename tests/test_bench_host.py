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
    rec = {"kernel_sha": "abc", "read_bytes_per_launch": 1000.4, "write_bytes_per_launch": 20.2,
           "clock_hz": 2.2e9}
    (prof / "qsa_prefill_kernel_w_traffic.json").write_text(json.dumps(rec))
    (prof / "qsa_prefill_kernel_old_traffic.json").write_text(json.dumps(
        {"kernel_sha": "abc", "fetch_bytes_per_launch": 1.0, "write_bytes_per_launch": 2.0}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", "abc") == rec
    assert bench.measured_traffic("w", "abd") is None
    assert bench.measured_traffic("other", "abc") is None
    assert bench.measured_traffic("old", "abc") is None  # a record without request-size read bytes


def test_roofline_is_the_l2_return_path():
    """Gathered bytes over the L2 -> CU return path's peak (16 KiB per clock at
    2.4 GHz), with past-L2 traffic set against the HBM peak."""
    assert bench.L2_CU_PEAK_GBPS == pytest.approx(39321.6)
    gathered, secs = 133_146_083_328, 5.9e-3
    roof, past = bench.roofline_records(gathered, secs, None)
    assert roof["bound"] == "l2" and roof["unit"] == "GB/s" and past is None and roof["traffic"] is None
    assert roof["achieved"] == pytest.approx(gathered / secs / 1e9, abs=0.1)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4) and 0 < roof["frac"] < 1
    rec = {"read_bytes_per_launch": 11.0e9, "write_bytes_per_launch": 0.4e9, "clock_hz": 2.14e9}
    roof, past = bench.roofline_records(gathered, secs, rec)
    assert roof["traffic"] == 11_400_000_000
    assert roof["frac_at_profiled_clock"] == pytest.approx(gathered / secs / (16384 * 2.14e9), abs=1e-4)
    assert past["GBps"] == pytest.approx(11.4e9 / secs / 1e9, abs=0.1)
    assert past["frac_of_hbm_peak"] == pytest.approx(11.4e9 / secs / 8e12, abs=1e-4)


def test_committed_profiles_name_their_library():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.endswith("_traffic.json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", name)))
            assert len(rec["kernel_sha"]) == 16
            assert rec.get("read_bytes_per_launch", rec.get("fetch_bytes_per_launch", 0)) > 0
            assert all("bench.py" in c for c in rec["commands"])


def test_oracle_worker_count_is_reported():
    from oracle import pool
    assert 1 <= pool.default_workers() <= pool.MAX_WORKERS
    assert pool.default_workers() <= pool.affinity_cpus()


def test_kernel_occupancy_rule():
    """bench.py mirrors the library's launch rule to run the gather probe at
    the kernel's waves per CU: one 4-wave block per CU for caches of 81,920
    rows or more with 32,768 items or more."""
    from qsa_inputs import get_config
    waves = {n: bench.kernel_waves_per_cu(get_config(n)) for n in range(1, 14)}
    assert waves[4] == waves[3] == waves[10] == waves[8] == waves[6] == 8
    assert waves[5] == waves[13] == 4
    assert waves[11] is None and waves[12] is None
    src = open(os.path.join(ROOT, "top_sparse_attention_qsa_amd", "csrc", "qsa_prefill.hip")).read()
    assert f"kOneBlockRows = {bench.ONE_BLOCK_ROWS};" in src
    assert f"kOneBlockItems = {bench.ONE_BLOCK_ITEMS};" in src


def test_probe_output_is_parsed():
    line = ("gather probe: rows 8192 (4.2 MB), 8 waves/CU, 16 loads in flight per wave (128 KB per CU): "
            "median 1.086 ms of 5, 24.72 TB/s\n")
    assert bench.parse_probe(line) == pytest.approx(24720.0)
    assert bench.parse_probe("nothing") is None


def test_parity_record_applies_the_bar():
    """bench.py compares the GPU's outputs on the CPU baseline's rows with the
    oracle's: bf16 rounding of the exact value passes, an error of 0.02
    fails, and an empty row must be +0.0 with lse = -inf on both sides."""
    import numpy as np
    from qsa_inputs import f32_to_bf16_bits
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((5, 3, 256)) * 3
    ref_lse = rng.standard_normal((5, 3))
    ref_lse[4] = -np.inf
    ref[4] = 0.0
    bits = f32_to_bf16_bits(ref.astype(np.float32))
    lse = ref_lse.astype(np.float32)
    rec = bench.parity_record(np.arange(5), ref, ref_lse, bits, lse)
    assert rec["within_bar"] and rec["outside_bar"] == 0 and rec["rows_checked"] == 5
    assert 0 < rec["max_abs_out"] <= 2 ** -4 and rec["max_abs_lse"] < 1e-6  # half an ulp reaches 2^-5 at |o| >= 8
    bad = f32_to_bf16_bits((ref + 0.02 * (np.abs(ref) < 1)).astype(np.float32))
    assert not bench.parity_record(np.arange(5), ref, ref_lse, bad, lse)["within_bar"]
    lse_bad = lse.copy()
    lse_bad[4, 0] = 0.0
    assert not bench.parity_record(np.arange(5), ref, ref_lse, bits, lse_bad)["within_bar"]

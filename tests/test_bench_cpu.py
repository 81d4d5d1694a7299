"""CPU checks of the benchmark's host side: it refuses more than one GPU, its
count of computed block scores agrees with the oracle's output, and stored
HBM traffic figures are reported only for the sources they were taken on."""
import dataclasses
import json
import os
import subprocess
import sys

import pytest
import torch

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


# the tiny configuration and a spread of random cases (MXFP4 left out: its
# E8M0 scales can encode NaN, which the count below would not see as a score)
CASES = [synth.config_case(0)] + synth.random_cases(16)


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c.name for c in CASES])
def test_score_count_matches_oracle(idx):
    # With no local_mask, an entry of the oracle's output is finite exactly
    # when its block has a visible key (the inputs are finite): the count the
    # benchmark's block scores/s is based on.
    c = dataclasses.replace(CASES[idx], init_blocks=0, local_blocks=0)
    out = oracle.index_score_case(c)
    assert bench.workload_stats(c)["scores"] == int(torch.isfinite(out).sum())


def test_traffic_only_for_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({
        "now": {"kernel_hash": bench.kernel_source_hash(), "bytes_per_launch": 123},
        "old": {"kernel_hash": "0" * 16, "bytes_per_launch": 5}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("now") == 123
    assert bench.measured_traffic("old") is None
    assert bench.measured_traffic("absent") is None


def test_host_cpu_reports_the_share_it_uses(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    h = bench.host_cpu()
    for k in ("nproc", "affinity", "cgroup_cpus", "omp_num_threads", "cpu_model",
              "cores_available"):
        assert k in h
    assert h["omp_num_threads"] == 3
    assert 1 <= h["cores_available"] <= min(3, h["affinity"])
    monkeypatch.delenv("OMP_NUM_THREADS")
    h = bench.host_cpu()
    assert h["omp_num_threads"] is None
    assert h["cores_available"] <= h["affinity"] <= (h["nproc"] or h["affinity"])


def test_cpu_baseline_legs():
    import argparse
    args = argparse.Namespace(cpu_rows=2)
    host = dict(bench.host_cpu(), cores_available=2)
    tiny = synth.config_case(0)
    r = bench.cpu_baseline_leg(tiny, bench.workload_stats(tiny), args, host)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["value"] > 0
    assert r["host"]["cpu_model"] == host["cpu_model"] and not r["extrapolated"]
    # the whole tiny example on one core too: 512 block scores
    assert r["single_core"]["cores"] == 1 and not r["single_core"]["extrapolated"]
    assert "512 block scores" in r["single_core"]["sample"]
    pre = synth.config_case(2)
    r = bench.cpu_baseline_leg(pre, bench.workload_stats(pre), args, host)
    assert r["extrapolated"] and r["value"] > 0 and "2 whole rows" in r["sample"]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c.name for c in CASES])
def test_per_token_visible_blocks_sum_to_the_score_count(idx):
    c = CASES[idx]
    assert int(bench.visible_blocks_per_token(c).sum()) * c.Hq == bench.workload_stats(c)["scores"]


def test_decode_batch_stats_agree_with_workload_stats():
    # the batch-scaling mode counts its work in closed form; on the bf16
    # decode workload itself (same distribution, B = 64) it must agree with
    # the general per-request count
    c = synth.config_case(1)
    want = bench.workload_stats(c)
    got = bench.decode_batch_stats(c.kv_len.numpy(), c.Hq, c.Hkv, c.D, c.block_size,
                                   c.max_blocks, 2)
    for key in ("scores", "out_entries", "flops", "bytes", "k_bytes", "q_bytes", "out_bytes"):
        assert got[key] == want[key], key

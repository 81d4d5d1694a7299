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

"""Host-side logic of bench.py that needs no GPU: the one-GPU rule, the loud failure
without a GPU, and the rule that a committed HBM traffic reading only applies to the
kernel sources it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=600)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run(env=env)
    assert r.returncode == 2


def test_no_gpu_fails_loudly():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "GPU" in r.stderr
    assert not r.stdout.strip().startswith("{")  # no result line without the GPU path


def test_committed_traffic_readings_match_the_sources():
    """Every committed reading was taken on the sources as they are (so the bench reports it)."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    for key, w in rec["workloads"].items():
        assert bench.source_sha256(w["sources"]) == w["source_sha256"], key
        workload, _, which = key.partition(":")
        assert bench.measured_traffic(workload, which or "fwd") == int(w["bytes"])


def test_traffic_reading_is_dropped_when_a_source_changes(tmp_path, monkeypatch):
    csrc = tmp_path / "selective_state_space_22_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel v1")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"workloads": {"w": {"bytes": 1234, "sources": ["k.hip"], "source_sha256": bench.source_sha256(["k.hip"])}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w") == 1234
    (csrc / "k.hip").write_text("kernel v2")
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("other") is None

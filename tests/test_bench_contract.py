"""Host-side checks of bench.py that need no GPU: it refuses more than one GPU
before touching a device, and it reports the committed HBM byte counters only
while the sources they were taken for are unchanged."""
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          env=env, timeout=120)


def test_refuses_more_than_one_gpu():
    res = _run(["--gpus", "2"])
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_refuses_a_multi_rank_launch():
    res = _run([], {"WORLD_SIZE": "2"})
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_traffic_record_matches_the_current_sources():
    with open(os.path.join(ROOT, "profiles", "paged_decode_traffic.json")) as f:
        rec = json.load(f)
    for src in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, src)), src
    got = bench.measured_traffic()
    assert got == rec["bytes_per_launch"]
    # traffic is within a few percent of the algorithmic bytes of the call
    assert 1.0 <= got / rec["algorithmic_bytes"] < 1.05


def test_traffic_is_withheld_once_a_source_changes(tmp_path, monkeypatch):
    with open(os.path.join(ROOT, "profiles", "paged_decode_traffic.json")) as f:
        rec = json.load(f)
    os.makedirs(tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "profiles", "paged_decode_traffic.json"), tmp_path / "profiles")
    for src in rec["sources"]:
        os.makedirs(os.path.dirname(tmp_path / src), exist_ok=True)
        shutil.copy(os.path.join(ROOT, src), tmp_path / src)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.measured_traffic() == rec["bytes_per_launch"]
    with open(tmp_path / rec["sources"][0], "a") as f:
        f.write("\n// edited\n")
    assert bench.measured_traffic() is None


def test_prefill_traffic_records_are_consistent():
    """Each prefill traffic record names its kernels' sources; while they are unchanged
    bench.py reports the recorded bytes, which exceed the algorithmic ones."""
    for row in ("prefill", "causal2k"):
        spec = bench.TRAFFIC_ROWS[row]
        with open(os.path.join(ROOT, "profiles", spec["file"])) as f:
            rec = json.load(f)
        assert rec["sources"] == spec["sources"]
        assert set(rec["fetch_kib"]) == set(spec["kernels"])
        got = bench.measured_traffic(row)
        if got is not None:
            assert got == rec["bytes_per_launch"]
            assert got > rec["algorithmic_bytes"]

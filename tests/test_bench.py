"""bench.py's host logic (no GPU needed): the one-GPU contract, the headline
workload, and the gating of the counter-derived HBM traffic by source hashes."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import fa_inputs  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_workload_is_the_causal_n8192_forward():
    w = fa_inputs.WORKLOADS[bench.MAIN]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (2, 32, 8192, 128, "bf16", True)
    assert bench.PEAK_TFLOPS["bf16"] == 2516.6 and bench.PEAK_TFLOPS["fp8"] == 5033.2


def test_traffic_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    """measured_traffic() returns the committed figure while the kernel's
    sources hash as recorded, and None once they differ (or nothing was
    recorded for that workload and stage)."""
    (tmp_path / "profiles").mkdir()
    current = {"fwd": "a" * 64, "dq": "b" * 64, "dkdv": "c" * 64}
    recorded = {"workloads": {"w": {"stages": {
        "fwd": {"source_sha256": "a" * 64, "bytes_per_launch": 123.0},
        "dq": {"source_sha256": "0" * 64, "bytes_per_launch": 456.0}}}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(recorded))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda stage: current[stage])
    assert bench.measured_traffic("w", "fwd") == 123.0
    assert bench.measured_traffic("w", "dq") is None     # taken on other sources
    assert bench.measured_traffic("w", "dkdv") is None   # nothing recorded
    assert bench.measured_traffic("other", "fwd") is None


def test_source_hash_covers_every_listed_file():
    for stage, files in bench.STAGE_SOURCES.items():
        for rel in files:
            assert os.path.exists(os.path.join(ROOT, "exact_io_aware_11_amd", rel)), (stage, rel)
        assert len(bench.source_hash(stage)) == 64

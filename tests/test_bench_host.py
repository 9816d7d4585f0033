"""Host-side logic of bench.py (CPU only): argument checks that end the run
before any device work, and the rule that the committed HBM-traffic figure is
reported only while the kernel source it was measured on is unchanged."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, env=env, timeout=120)


def test_more_than_one_gpu_is_refused_before_device_work():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, cwd=ROOT, env=env, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_unknown_variant_is_refused():
    r = _run("--variants", "backward,nonsense")
    assert r.returncode == 2
    assert "nonsense" in r.stderr


def test_every_variant_name_is_known():
    assert set(bench.VARIANTS) == {"options", "slices", "backward", "rmsnorm", "topk20",
                                   "long_rollout", "decode"}


def test_traffic_is_reported_only_for_the_profiled_source(monkeypatch):
    digest = bench.kernel_source_digest()
    assert len(digest) == 16 and all(c in "0123456789abcdef" for c in digest)
    text = open(bench.TRAFFIC_FILE).read()
    assert "kernel_source_sha256_16:" in text and "hbm_bytes_per_launch:" in text
    # a different kernel source: the committed counters no longer describe it
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.measured_traffic() is None


def test_traffic_figure_is_read_when_the_source_matches(monkeypatch, tmp_path):
    f = tmp_path / "traffic.md"
    f.write_text("kernel_source_sha256_16: 0123456789abcdef\n\nhbm_bytes_per_launch: 7.5e+09\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0123456789abcdef")
    assert bench.measured_traffic() == pytest.approx(7.5e9)

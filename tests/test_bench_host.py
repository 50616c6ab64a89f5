"""Host logic of bench.py (CPU): the one-GPU guard, the whole-window step
count and the guard that reports the flush's HBM traffic only for the
kernel sources it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("k,w,want", [(20, 16, 32), (32, 16, 32), (1, 16, 16), (0, 16, 16),
                                      (64, 32, 64), (65, 32, 96), (7, 1, 7), (160, 16, 160)])
def test_timed_steps_are_whole_windows(k, w, want):
    got = bench.timed_steps(k, w)
    assert got == want and got % w == 0 and got >= max(k, w)


def test_traffic_reported_only_for_the_measured_sources(monkeypatch):
    digest = bench.flush_src_digest()
    assert digest == bench.flush_src_digest() and len(digest) == 64
    for f in bench.FLUSH_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "ssm_decode_amd", "csrc", f)), f
    monkeypatch.setitem(bench.TRAFFIC, "probe", {"bytes": 123, "src_sha256": digest})
    assert bench.flush_traffic("probe") == 123
    monkeypatch.setitem(bench.TRAFFIC, "probe", {"bytes": 123, "src_sha256": "0" * 64})
    assert bench.flush_traffic("probe") is None
    assert bench.flush_traffic("no_such_workload") is None


def test_read_traffic_reported_only_for_the_measured_sources(monkeypatch):
    digest = bench.read_src_digest()
    assert len(digest) == 64 and digest != bench.flush_src_digest()
    for f in bench.READ_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "ssm_decode_amd", "csrc", f)), f
    assert "sk_read.hpp" in bench.READ_SOURCES
    monkeypatch.setitem(bench.TRAFFIC_READ, "probe", {"bytes": 7, "src_sha256": digest})
    assert bench.read_traffic("probe") == 7
    monkeypatch.setitem(bench.TRAFFIC_READ, "probe", {"bytes": 7, "src_sha256": "0" * 64})
    assert bench.read_traffic("probe") is None
    assert bench.read_traffic("no_such_workload") is None
    # the stored figures are for the sources as they stand
    for name in ("m2_b320", "gdn_b256", "kda_b256"):
        assert bench.read_traffic(name) == bench.TRAFFIC_READ[name]["bytes"]


def test_cpu_model_is_named():
    m = bench.cpu_model()
    assert isinstance(m, str) and m

"""Host-side checks of bench.py (no GPU needed): the one-GPU refusal and the
rule that a traffic figure from a committed counter summary is reported only
while the kernel sources it was taken on are unchanged."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_source_digest_follows_the_sources(tmp_path):
    b = _bench()
    d1 = b.kernel_sources_digest(["bwd.hip", "sla_device.h"])
    assert d1 == b.kernel_sources_digest(["bwd.hip", "sla_device.h"])
    assert d1 != b.kernel_sources_digest(["attn_fwd.hip", "sla_device.h"])
    assert d1 != b.kernel_sources_digest(["bwd.hip"])


def test_traffic_only_for_the_profiled_sources(tmp_path, monkeypatch):
    b = _bench()
    (tmp_path / "profiles").mkdir()
    rec = {"kernel": "k", "source_digest": "abc123", "hbm_bytes_per_launch": 12345}
    (tmp_path / "profiles" / "traffic_k_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.traffic_from_profile("k", "wl", "abc123") == 12345
    assert b.traffic_from_profile("k", "wl", "stale") is None          # kernel changed since
    assert b.traffic_from_profile("other", "wl", "abc123") is None     # never profiled

"""Host-side pieces of bench.py (CPU): the counter-traffic record is used only for the kernel
and workload it was taken on and only while every source it names is byte-for-byte the same;
bench.py refuses more than one GPU."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_record_tracks_its_sources(tmp_path, monkeypatch):
    b = _bench()
    (tmp_path / "a.hip").write_text("kernel a\n")
    (tmp_path / "b.h").write_text("helper b\n")
    h = hashlib.sha256()
    for f in ("a.hip", "b.h"):
        h.update((tmp_path / f).read_bytes())
    rec = dict(kernel="k", workload="w", hbm_bytes_per_launch=1234, sources=["a.hip", "b.h"],
               sources_sha256=h.hexdigest())
    path = tmp_path / "rec.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "TRAFFIC_RECORD", str(path))
    assert b.measured_traffic("k", "w") == 1234
    assert b.measured_traffic("k", "other workload") is None
    assert b.measured_traffic("other kernel", "w") is None
    (tmp_path / "b.h").write_text("helper b, edited\n")          # any source changed
    assert b.measured_traffic("k", "w") is None
    (tmp_path / "b.h").unlink()                                  # a source missing
    assert b.measured_traffic("k", "w") is None
    path.write_text(json.dumps(dict(rec, sources=[])))           # a record naming no source
    assert b.measured_traffic("k", "w") is None


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)

"""bench.py's command line on the host: more than one GPU is refused with a
message and exit status 2 before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_traffic_record_goes_stale_with_its_headers(tmp_path, monkeypatch):
    """A committed HBM-traffic record counts only while its kernel source and
    every header it lists hash as they did when the counters were taken."""
    import hashlib
    import json
    sys.path.insert(0, ROOT)
    import bench
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_bytes(b"kernel")
    (tmp_path / "h.h").write_bytes(b"header")
    sha = hashlib.sha256(b"kernel" + b"header").hexdigest()[:16]
    rec = {"workload": "w", "source": "k.hip", "headers": ["h.h"], "source_sha256_16": sha,
           "traffic_bytes": 123}
    (tmp_path / "profiles" / "w.md").write_text("```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w") == 123
    assert bench.measured_traffic("other") is None
    (tmp_path / "h.h").write_bytes(b"header, changed")
    assert bench.measured_traffic("w") is None

"""bench.py's command-line contract on the host (no GPU needed): more than
one GPU is refused with a message before anything touches a device, and
the HBM-traffic figure it reports comes from the committed profile only
while that profile was taken on the current kernel sources."""

import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_cli_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_traffic_is_tied_to_the_profiled_sources(tmp_path):
    b = _bench_module()
    with open(b.TRAFFIC_FILE.format("wan")) as f:
        t = json.load(f)
    assert t["workload"] == "wan" and len(t["kernel_source_sha256_16"]) == 16
    # A profile taken on other sources, or for another workload, gives no figure.
    stale = dict(t, kernel_source_sha256_16="0" * 16)
    (tmp_path / "stale").mkdir()
    (tmp_path / "stale" / "wan.json").write_text(json.dumps(stale))
    b.TRAFFIC_FILE = str(tmp_path / "stale" / "{}.json")
    assert b.traffic_per_launch("wan") is None
    (tmp_path / "good").mkdir()
    (tmp_path / "good" / "wan.json").write_text(json.dumps(t))
    (tmp_path / "good" / "hunyuan.json").write_text(json.dumps(t))  # names the wrong workload
    b.TRAFFIC_FILE = str(tmp_path / "good" / "{}.json")
    want = b.traffic_per_launch("wan") if t["kernel_source_sha256_16"] == b.kernel_source_hash() else None
    assert b.traffic_per_launch("hunyuan") is None
    if want is not None:
        assert want > 0

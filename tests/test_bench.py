"""CPU checks of bench.py's host logic: it refuses more than one GPU, and its
helpers name profiles and accept traffic figures only for the current kernel
source."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_name():
    assert bench.traffic_name("f16_8192", "kblock", "kn") == "f16_8192"
    assert bench.traffic_name("f16_8192", "row", "nk") == "f16_8192_row_nk"


def test_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_w.json").write_text(json.dumps({"kernel_src_hash": "abc", "gemm_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("w", "abc") == 123
    assert bench.load_traffic("w", "abd") is None
    assert bench.load_traffic("missing", "abc") is None


def test_region_bookkeeping():
    bench.CALLS["gemm"] = 5
    bench.region_open("r", "gemm")
    bench.CALLS["gemm"] += 3
    bench.region_close("r")
    assert bench.REGIONS["r"] == {"calls_of": "gemm", "first": 5, "end": 8}

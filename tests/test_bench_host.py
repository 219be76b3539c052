"""Host-side behaviour of bench.py that needs no GPU: the one-GPU rule and
the rule that the counter-based traffic figure is reported only for the
kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    rec = {"bytes_per_launch": 12345, "kernel_source_sha256": bench.kernel_source_digest()}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() == 12345
    rec["kernel_source_sha256"] = "0" * 64  # taken on other sources
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None
    f.write_text("not json")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_source_digest_covers_the_gemm_sources(tmp_path, monkeypatch):
    # the digest changes with any byte of the GEMM kernel sources
    d0 = bench.kernel_source_digest()
    csrc = tmp_path / "sparse_moe_layer_06_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("gemm_mfma.hip", "device_common.hpp", "lmoe_internal.hpp"):
        with open(os.path.join(ROOT, "sparse_moe_layer_06_amd", "csrc", name), "rb") as fh:
            (csrc / name).write_bytes(fh.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_digest() == d0
    (csrc / "device_common.hpp").write_bytes((csrc / "device_common.hpp").read_bytes() + b"\n")
    assert bench.kernel_source_digest() != d0

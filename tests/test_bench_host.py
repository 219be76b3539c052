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


def test_source_digest_covers_the_gemm_code(tmp_path, monkeypatch):
    # the digest changes with the code of the GEMM kernel sources, not with
    # their comments or layout
    d0 = bench.kernel_source_digest()
    csrc = tmp_path / "sparse_moe_layer_06_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("gemm_mfma.hip", "device_common.hpp", "lmoe_internal.hpp"):
        with open(os.path.join(ROOT, "sparse_moe_layer_06_amd", "csrc", name), "rb") as fh:
            (csrc / name).write_bytes(fh.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_digest() == d0
    f = csrc / "device_common.hpp"
    base = f.read_bytes()
    f.write_bytes(base + b"\n// a comment\n/* another */\n")
    assert bench.kernel_source_digest() == d0
    f.write_bytes(base + b"\nconstexpr int kOneMore = 1;\n")
    assert bench.kernel_source_digest() != d0
    f.write_bytes(base.replace(b"static_for", b"static_for_", 1))
    assert bench.kernel_source_digest() != d0


def test_code_only_keeps_literals_and_drops_comments():
    src = 'int a = 1; // x\n/* y\n z */ const char* s = "//not a comment"; char c = \'"\';\n'
    assert bench.code_only(src) == 'int a = 1; const char* s = "//not a comment"; char c = \'"\';'


def test_oracle_timing_runs_single_threaded_on_host_inputs():
    # the CPU-baseline leg: the oracle on a token sample, BLAS limited to one thread
    import numpy as np

    from sparse_moe_layer_06_amd import synth
    cfg = synth.CONFIGS["tiny_f32"]
    inp = synth.make_inputs(cfg, 0, "cpu")
    dt = bench.oracle_seconds(cfg, inp, np.arange(8), synth, threads=1)
    assert dt > 0.0


def test_expert_gemm_bytes_count_weights_once_and_the_rows():
    from sparse_moe_layer_06_amd import synth
    C = synth.CONFIGS
    # mid: 128 experts of 1024 x 1024 bf16, 16384 rows of 1024 in and 1024 out
    assert bench.grouped_bytes_per_launch(C["mid_bf16"]) == 128 * 1024 * 1024 * 2 + 16384 * 2048 * 2
    # NVFP4: 4.5 bits per weight with 1-D scale blocks
    nv = C["prefill_nvfp4"]
    assert bench.grouped_bytes_per_launch(nv) == 512 * 2048 * 2048 * 9 / 16 + 8192 * 22 * 4096 * 2
    # skewed routing touches an unknown set of experts: no figure
    assert bench.grouped_bytes_per_launch(C["decode_bf16_zipf"]) is None

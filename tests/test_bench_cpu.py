"""bench.py's host logic without a GPU: the one-GPU refusal, the workload
registry, and the measured-traffic lookup (valid only while the sources of an
op's kernels are unchanged)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_workload_registry():
    # the default workload and every documented alternative are registered
    for name in ("dsv3_moe_mxfp8", "qwen3_moe_nvfp4", "qwen3_moe_nvfp4_bwd_hp", "qwen3_moe_nvfp4_bwd_deq",
                 "qwen3_moe_nvfp4_bwd_fp4", "mxfp8_quant", "requant_sr", "roundtrip", "hbm_copy"):
        assert name in bench.WORKLOADS, name
    # the default run also measures these, after the headline workload
    assert set(bench.SECONDARY) <= set(bench.WORKLOADS)
    assert "dsv3_moe_mxfp8" not in bench.SECONDARY


def test_kernel_source_digest_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "block_scaled_precision_token_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("int f(int x) {  // one\n  return x + 1; /* two */ }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    (csrc / "a.hip").write_text("int f(int x)\n{\n    // changed comment\n    return x + 1;\n}\n")
    assert bench.kernel_source_digest() == d0
    (csrc / "a.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_digest() != d0


def test_traffic_table_entries_name_registered_ops():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        pytest.skip("no traffic table")
    table = json.load(open(path))
    assert table["calibration"]["FETCH_SIZE"] > 0 and table["calibration"]["WRITE_SIZE"] > 0
    for key, ent in table["ops"].items():
        wl, op = key.split("/")
        assert wl in bench.WORKLOADS, key
        assert ent["bytes_per_launch"] == ent["fetch_bytes"] + ent["write_bytes"] or \
            abs(ent["bytes_per_launch"] - ent["fetch_bytes"] - ent["write_bytes"]) <= 1, key
        assert len(ent["source_sha256"]) == 64
        # the lookup returns the stored bytes exactly when the op's sources still match
        current = bench.kernel_source_digest(bench.kernel_sources_of(op))
        got = bench.measured_traffic(wl, op)
        assert got == (ent["bytes_per_launch"] if ent["source_sha256"] == current else None), key

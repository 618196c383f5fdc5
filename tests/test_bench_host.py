"""Host-side behaviour of bench.py (no GPU needed): the one-GPU refusal and
the HBM-traffic lookup, which is only trusted while the kernel sources still
match the digest the counters were taken with."""

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


def test_traffic_lookup_follows_the_source_digest(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()
    assert len(digest) == 16 and digest == bench.kernel_source_digest()
    table = {"dense_fprop:gemm_blockscaled": {"bytes_per_launch": 123, "source_digest": digest},
             "decode:grouped_gemm_decode": {"bytes_per_launch": 456, "source_digest": "0" * 16}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(table))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("gemm_blockscaled", "dense_fprop") == 123
    assert bench.measured_traffic("grouped_gemm_decode", "decode") is None      # stale digest
    assert bench.measured_traffic("quant_act_1x128", "dense_fprop") is None     # not measured
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("gemm_blockscaled", "dense_fprop") is None


def test_committed_traffic_table_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        table = json.load(f)
    assert table
    for key, ent in table.items():
        workload, kernel = key.split(":")
        assert workload in bench.WORKLOADS
        assert abs(ent["bytes_per_launch"] - ent["fetch_bytes"] - ent["write_bytes"]) <= 1   # each rounded
        assert len(ent["source_digest"]) == 16


def test_percentile_interpolates():
    xs = [4.0, 1.0, 3.0, 2.0]
    assert bench.percentile(xs, 0.0) == 1.0 and bench.percentile(xs, 1.0) == 4.0
    assert bench.percentile(xs, 0.5) == 2.5
    assert abs(bench.percentile(list(range(11)), 0.1) - 1.0) < 1e-12


def test_default_run_covers_every_configuration():
    # the headline is the dense Fprop; the default run adds the tiny Fprop,
    # the grouped MoE GEMMs, the decode-shaped grouped GEMM and the backward pair
    names = [wl for _, wl in bench.EXTRA_CONFIGS]
    assert names == ["tiny_fprop", "moe", "decode", "backward"]
    assert all(wl in bench.WORKLOADS for wl in names)

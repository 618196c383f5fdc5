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


def test_cast_ceiling_is_the_plain_cast_of_the_same_tensor(monkeypatch):
    # the quantizers' streaming ceiling: PyTorch's BF16 -> E4M3 cast of copies
    # of the input, as many as _rotations asks for (here 3, to keep it small)
    import torch
    copies = []
    monkeypatch.setattr(bench, "_rotations", lambda nbytes: copies.append(nbytes) or 3)
    x = (torch.randn((64, 256)) * 3).to(torch.bfloat16)
    run = bench._cast_ceilings(torch, torch.device("cpu"), {"quant_act_1x128": x})["quant_act_1x128"]
    assert copies == [x.numel() * 3]          # BF16 in, one code byte out
    want = x.to(torch.float8_e4m3fn).view(torch.uint8)
    outs = [run(i) for i in range(4)]
    for got in outs:
        assert got.dtype == torch.float8_e4m3fn and torch.equal(got.view(torch.uint8), want)
    assert outs[3].data_ptr() == outs[0].data_ptr() != outs[1].data_ptr()   # cycles through 3 outputs


def test_rotations_exceed_the_infinity_cache():
    for nbytes in (1 << 20, 88_000_000, 300_000_000, 2_000_000_000):
        n = bench._rotations(nbytes)
        assert n >= 2 and n * nbytes >= 600e6


def test_clock_summary_drops_the_stale_leading_readings():
    # the SMI refreshes about once a second: readings from before the load
    # repeat until the first refresh and are dropped once a new one arrives
    s = bench.clock_summary([95.0, 95.0, 95.0, 1969.0, 1969.0, 1950.0], "test")
    assert s["median_mhz"] == 1969.0 and s["min_mhz"] == 1950.0 and s["samples"] == 3 and s["stale_dropped"] == 3
    s = bench.clock_summary([2079.0] * 5)          # no refresh seen: every reading kept
    assert s["median_mhz"] == 2079.0 and s["samples"] == 5 and s["stale_dropped"] == 0
    assert bench.clock_summary([]) is None


def test_source_digest_ignores_comments_only():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    assert bench._code_only(code) == bench._code_only(code.replace("one more", "plus one").replace("block", "b"))
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))
    assert bench._code_only("a  =\n b;") == "a = b;"


def test_kernel_choice_reports_the_library_pick():
    import fp8_block_scaled_x1_amd as fb
    assert bench._kernel_choice(fb, 4096, 7168, 7168, fb.SCALE_BLOCK128) == \
        {"tile": [256, 224], "ring_depth": 3, "tail_tiles": 0}
    assert bench._kernel_choice(fb, 7168, 7168, 4096, fb.SCALE_ROW) == \
        {"tile": [256, 256], "ring_depth": 2, "tail_tiles": 16}

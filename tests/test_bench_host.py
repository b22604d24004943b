"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic byte counts its
roofline figures divide by, and the rocprofv3 summaries (copy calibration of the traffic counters,
traffic records tied to the kernel sources)."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_append_bytes_per_token_head():
    # bf16 K and V in (2 x 128 x 2 B), codes out (2 x 64 B INT4, 2 x 32 B INT2), a float32 scale and
    # zero per tensor (16 B), plus each token's int64 slot
    assert bench.append_bytes(1, 1, 4) == 656 + 8
    assert bench.append_bytes(1, 1, 2) == 592 + 8
    assert bench.append_bytes(65536, 8, 4) == 65536 * 8 * 656 + 65536 * 8


def test_decode_bytes_per_token_head():
    # codes and scale/zero of every attended token-head (144 B INT4, 80 B INT2), one block-table
    # entry per page, bf16 q and float32 out per query head, one context length per sequence
    lens = [16, 17]
    assert bench.decode_bytes(lens, 32, 8, 4, 16) == 33 * 8 * 144 + 3 * 4 + 2 * 32 * 128 * (2 + 4) + 2 * 4
    assert bench.decode_bytes([5], 8, 8, 2, 16) == 5 * 8 * 80 + 4 + 8 * 128 * 6 + 4
    assert bench.decode_bytes([0], 8, 8, 4, 16) == 8 * 128 * 6 + 4


def test_per_channel_bytes():
    # a page of 64 tokens of one KV head, INT2: per token 512 B in, 64 B of codes and two float32
    # token scales out; per page 2 x 2 x 128 float32 channel parameters and its int32 id
    assert bench.pc_write_bytes(64, 1, 2, 64) == 64 * (512 + 64 + 8) + 2048 + 4
    # decode over one complete page plus a 3-token bf16 tail, one KV head, 7 query heads
    got = bench.pc_decode_bytes([67], 7, 1, 2, 64)
    assert got == 64 * (64 + 8) + 2048 + 3 * 512 + 4 + 7 * 128 * 6 + 4


def _write_counter_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    mib256_kib = (256 << 20) // 1024
    for counter, copy_kib, kern_kib, sub in (("FETCH_SIZE", mib256_kib / 2, 1000.0, "f"),
                                              ("WRITE_SIZE", mib256_kib, 500.0, "w")):
        d = tmp_path / sub
        d.mkdir()
        rows = [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=512, Counter_Name=counter,
                     Counter_Value=7.0)]  # a set-up copy: not one of the last three
        rows += [dict(Dispatch_Id=2 + i, Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=131072,
                      Counter_Name=counter, Counter_Value=copy_kib) for i in range(3)]
        rows += [dict(Dispatch_Id=10 + i, Kernel_Name="void kvq::append_kernel<4, false, 7>(kvq::AppendArgs, long)",
                      Grid_Size=2097152, Counter_Name=counter, Counter_Value=kern_kib) for i in range(2)]
        _write_counter_csv(d / "run_counter_collection.csv", rows)
    text = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), "llama3_8b", "CMD")
    assert "FETCH_SIZE x 2.0000" in text and "WRITE_SIZE x 1.0000" in text
    rec = json.loads([ln for ln in text.splitlines() if ln.startswith(bench.TRAFFIC_TAG)][0][len(bench.TRAFFIC_TAG):])
    a = rec["append_kernel"]
    assert a["read_bytes"] == 1000 * 1024 * 2 and a["write_bytes"] == 500 * 1024
    assert a["bytes_per_launch"] == 1000 * 1024 * 2 + 500 * 1024
    assert a["grid"] == 2097152 and a["sources_sha256"] == bench.sources_sha256("append_kernel")


@pytest.mark.parametrize("matching", [True, False])
def test_stored_traffic_is_tied_to_the_sources(tmp_path, monkeypatch, matching):
    sha = bench.sources_sha256("append_kernel") if matching else "0" * 64
    rec = {"append_kernel": {"bytes_per_launch": 123456, "grid": 1, "read_bytes": 1, "write_bytes": 1,
                             "sources_sha256": sha}}
    path = tmp_path / "hbm_traffic_llama3_8b.md"
    path.write_text("# HBM traffic\n\n" + bench.TRAFFIC_TAG + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "traffic_file", lambda workload: str(path))
    assert bench.stored_traffic("llama3_8b", "append_kernel") == (123456 if matching else None)
    assert bench.stored_traffic("llama3_8b", "decode_mfma_kernel") is None


def test_ceiling_launch_shapes_match_the_kernels():
    # the append: one wave per (16-token tile, KV head) item, four waves per 256-thread workgroup,
    # 512 B read and 144 B (INT4) / 80 B (INT2) written per token-head, in 16-byte units
    assert bench.Ceiling.append_shape(65536, 8, 4) == (8192, 256, 32, 9)   # Llama-3-8B prefill
    assert bench.Ceiling.append_shape(32 * 512, 4, 2) == (1024, 256, 32, 5)  # one OScaR chunk
    assert bench.Ceiling.append_shape(17, 3, 4) == (2, 256, 32, 9)          # 2 tiles x 3 heads = 6 items


def test_decode_waves_follow_the_split_plan():
    # one wave per (split, sequence, KV head), the splits read back from the workspace size: the
    # three large workloads each fill 2,048 waves (16 / 64 / 16 splits per item)
    assert bench._decode_waves(16, 32, 8, 4097, 16) == 16 * 16 * 8
    assert bench._decode_waves(4, 64, 8, 32769, 16) == 64 * 4 * 8
    assert bench._decode_waves(32, 28, 4, 16385, 16) == 16 * 32 * 4
    assert bench._decode_waves(1, 8, 8, 512, 16) == 4 * 1 * 8   # 32 pages, 8 per split at least

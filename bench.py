#!/usr/bin/env python3
"""Benchmark of the rotated INT4 paged KV-cache hot path on one MI355X.

One step = the whole hot path over one batch of the Llama-3-8B-shaped layer (16 sequences x
4096 tokens, 32 query / 8 KV heads, head_dim 128, page size 16, Hadamard block 128, INT4):

  1. rotate-quantize-append of the 16 x 4096 prefill tokens (write path, all 8 KV heads),
  2. the decode step: rotate-quantize-append of one new token per sequence and paged decode
     attention over the 4097 tokens (read path), fused in one launch (kvq_decode_step).

Inputs are seeded synthetic bf16 tensors resident in HBM before timing starts. To keep the
256 MB Infinity Cache from serving reads, steps rotate over 4 copies of the prefill inputs and
14 copies of the cache (about 2 GB), and the attention of step i reads the cache copy written
seven steps earlier. Prints one JSON line (see the keys at the bottom).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged INT4 decode-attn & quant-append HBM GB/s (% of MI355X peak), tokens/s"
PEAK_HBM_GBPS = 8000.0
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak
N_INPUT_COPIES = 4
N_CACHE_COPIES = 14


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="llama3_8b")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=("tiny", "sweep", "llama2_70b", "oscar_int2"),
                   help="time only this record (with its measured ceilings, without the CPU oracle) and print it")
    p.add_argument("--no-sub-records", action="store_true",
                   help="time only the Llama-3-8B step (no tiny, sweep, Llama-2-70B and OScaR records, no ceilings)")
    p.add_argument("--decode-iters", type=int, default=200, help="extra decode-only launches for the decode roofline")
    p.add_argument("--counters", action="store_true",
                   help="short program for rocprofv3 --pmc passes: a 256 MiB calibration copy, then --steps steps")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="print the HBM traffic summary of two rocprofv3 --pmc runs of --counters")
    p.add_argument("--suite", action="store_true",
                   help="time every workload shape (tiny, batch sweep with and without rotation, the 80-layer "
                        "Llama-2-70B step, the chunked OScaR INT2 prefill, per-channel pages, several queries per "
                        "sequence) and print one JSON line each")
    p.add_argument("--suite-cpu", action="store_true", help="with --suite: also time the CPU oracle on small samples")
    p.add_argument("--suite-only", default="",
                   help="with --suite: run only these parts (comma list of tiny, sweep, llama2_70b, oscar, pc, multi_query)")
    p.add_argument("--summarize-sq", nargs=2, metavar=("INST_DIR", "CYCLE_DIR"),
                   help="print the SQ instruction-mix and wave-state summary of two rocprofv3 --pmc runs")
    p.add_argument("--summarize-kernel-stats", metavar="RUN_DIR",
                   help="print the kernel table of a rocprofv3 --kernel-trace --stats run as markdown")
    return p.parse_args()


def append_bytes(tokens: int, heads: int, bits: int, d: int = 128) -> int:
    """Algorithmic bytes of rotate-quantize-append: bf16 K+V read, codes + fp32 scale/zero
    written for K and V, plus the int64 slot of every token."""
    per_token_head = 2 * d * 2 + 2 * d * bits // 8 + 2 * 8
    return tokens * heads * per_token_head + tokens * 8


def decode_bytes(lens, num_q_heads: int, num_kv_heads: int, bits: int, page_size: int, d: int = 128) -> int:
    """Algorithmic bytes of one decode step: K/V codes + scale/zero of every attended token
    and KV head, the block-table entries read, bf16 q, fp32 out and the context lengths."""
    per_token_head = 2 * d * bits // 8 + 2 * 8
    toks = int(np.sum(lens))
    pages = int(np.sum((np.asarray(lens) + page_size - 1) // page_size))
    b = len(lens)
    return toks * num_kv_heads * per_token_head + pages * 4 + b * num_q_heads * d * (2 + 4) + b * 4


# ----------------------------------------------------------------------------- HBM traffic counters
#
# rocprofv3's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) do not count every byte the same way
# (FETCH_SIZE counts a 128-byte read as one 64-byte request), so each is scaled by the ratio it
# shows on a plain 256 MiB device copy in the same run. The traffic recorded for a kernel is tied
# to what it was built from - its source files and the compiler flags of its translation unit (the
# first file listed): once they change, the stored figure no longer applies.

CSRC = os.path.join(ROOT, "paged_decode_attention_amd", "csrc")
KERNEL_SOURCES = {
    "append_kernel": ["kvq_append.hip", "kvq_rotate_mfma.h", "kvq_mfma.h", "kvq_device.h", "kvq_launch.h", "kvq_fastdiv.h"],
    "decode_mfma_kernel": ["kvq_decode_mfma.hip", "kvq_decode.hip", "kvq_mfma.h", "kvq_device.h", "kvq_launch.h", "kvq_fastdiv.h"],
    "decode_merge_splits_kernel": ["kvq_decode_mfma.hip", "kvq_mfma.h", "kvq_device.h", "kvq_launch.h", "kvq_fastdiv.h"],
    "chunk_attention_kernel": ["kvq_chunk_attn.hip", "kvq_chunk.h", "kvq_mfma.h", "kvq_device.h", "kvq_launch.h", "kvq_fastdiv.h"],
}
CALIBRATION_BYTES = 256 << 20
TRAFFIC_TAG = "traffic-json: "


def sources_sha256(kernel: str) -> str:
    import hashlib
    from paged_decode_attention_amd import build as _build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.normpath(os.path.join(CSRC, f)), "rb") as fh:
            h.update(fh.read())
    tu = KERNEL_SOURCES[kernel][0]
    # the flags without the include directory (an absolute path that differs between checkouts)
    flags = [f for f in _build.CFLAGS + _build.EXTRA_CFLAGS.get(tu, []) if not os.path.isabs(f)]
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")


def stored_traffic(workload: str, kernel: str):
    """Measured HBM bytes per launch of ``kernel``, or None if absent or taken on other sources."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith(TRAFFIC_TAG):
                rec = json.loads(line[len(TRAFFIC_TAG):]).get(kernel)
                if rec and rec["sources_sha256"] == sources_sha256(kernel):
                    return rec["bytes_per_launch"]
    return None


def _short_kernel_name(name: str) -> str:
    for k in list(KERNEL_SOURCES) + ["copyBuffer"]:
        if k in name:
            return k
    return name.split("(")[0][-60:]


def _counter_rows(run_dir: str, counter: str):
    """(kernel, grid, value) per dispatch, in dispatch order."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), _short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]),
                                 float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    return [r[1:] for r in sorted(rows)]


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, command: str) -> str:
    per = {}
    factors = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(run_dir, counter)
        # --counters issues its three calibration copies after every set-up copy and before the
        # steps, which copy nothing: they are the last three copy dispatches of the run
        cal = [v for k, g, v in rows if k == "copyBuffer"][-3:]
        factors[counter] = CALIBRATION_BYTES / (1024.0 * float(np.median(cal)))
        for k, g, v in rows:
            if k in KERNEL_SOURCES:
                per.setdefault((k, g), {}).setdefault(counter, []).append(v)
    lines = ["| kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---|---|---|---|---|---|"]
    rec = {}
    for (k, g), cs in sorted(per.items()):
        fk = float(np.median(cs.get("FETCH_SIZE", [0.0])))
        wk = float(np.median(cs.get("WRITE_SIZE", [0.0])))
        rd = fk * 1024 * factors["FETCH_SIZE"]
        wr = wk * 1024 * factors["WRITE_SIZE"]
        lines.append(f"| {k} | {g} | {len(cs.get('FETCH_SIZE', []))} | {fk:.1f} | {wk:.1f} | {rd / 1e6:.2f} | "
                     f"{wr / 1e6:.2f} |")
        # the record keeps the largest grid of each kernel (the prefill append, the full decode)
        if k not in rec or g > rec[k]["grid"]:
            rec[k] = {"grid": g, "bytes_per_launch": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr),
                      "sources_sha256": sources_sha256(k)}
    head = [f"# HBM traffic per launch, {workload}", "",
            f"Command (twice, once per counter): `{command}`", "",
            f"Calibration: a {CALIBRATION_BYTES >> 20} MiB device copy (__amd_rocclr_copyBuffer) in the same run reads "
            f"FETCH_SIZE x {factors['FETCH_SIZE']:.4f} and writes WRITE_SIZE x {factors['WRITE_SIZE']:.4f} of its true "
            "size; every kernel's counters are scaled by these factors (median over dispatches).", ""]
    return "\n".join(head + lines + ["", TRAFFIC_TAG + json.dumps(rec, sort_keys=True), ""])


SQ_INSTS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_MFMA", "SQ_INSTS_VMEM_RD")
SQ_CYCLES = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA",
             "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM")


def summarize_sq(inst_dir: str, cycle_dir: str, workload: str) -> str:
    """Instruction mix per wave and the split of wave-cycles between issuing and waiting, from two
    rocprofv3 --pmc runs of bench.py --counters (median over the dispatches of each kernel and grid)."""
    def per_dispatch(run_dir, counters):
        vals = {}
        for c in counters:
            seen = {}
            for k, g, v in _counter_rows(run_dir, c):
                seen.setdefault((k, g), []).append(v)
            for key, vs in seen.items():
                vals.setdefault(key, {})[c] = vs
        return vals
    inst = per_dispatch(inst_dir, SQ_INSTS + ("SQ_WAVE_CYCLES",))
    cyc = per_dispatch(cycle_dir, SQ_CYCLES + ("SQ_WAVE_CYCLES",))
    med = lambda xs: float(np.median(xs))  # noqa: E731
    lines = ["| kernel | grid | waves | VALU / wave | SALU / wave | MFMA / wave | VMEM reads / wave |",
             "|---|---|---|---|---|---|---|"]
    for (k, g), c in sorted(inst.items()):
        if k not in KERNEL_SOURCES:
            continue
        w = med(c["SQ_WAVES"])
        lines.append(f"| {k} | {g} | {w:.0f} | {med(c['SQ_INSTS_VALU']) / w:.0f} | {med(c['SQ_INSTS_SALU']) / w:.0f} | "
                     f"{med(c['SQ_INSTS_MFMA']) / w:.0f} | {med(c['SQ_INSTS_VMEM_RD']) / w:.1f} |")
    lines += ["", "Share of wave-cycles (SQ_WAVE_CYCLES) per state:", "",
              "| kernel | grid | " + " | ".join(x[3:].lower() for x in SQ_CYCLES) + " |",
              "|---|---|" + "---|" * len(SQ_CYCLES)]
    for (k, g), c in sorted(cyc.items()):
        if k not in KERNEL_SOURCES:
            continue
        wc = med(c["SQ_WAVE_CYCLES"])
        lines.append(f"| {k} | {g} | " + " | ".join(f"{med(c[x]) / wc:.3f}" for x in SQ_CYCLES) + " |")
    cmd = ("rocprofv3 --pmc {counters} --output-format csv -d DIR -o run -- python3 bench.py --counters "
           f"--workload {workload} --steps 3 --warmup 0")
    head = [f"# Instruction mix and wave states, {workload}", "",
            "Commands (two runs, one per counter set; at most 8 SQ counters per run):", "",
            "- `" + cmd.format(counters=" ".join(SQ_INSTS + ("SQ_WAVE_CYCLES",))) + "`",
            "- `" + cmd.format(counters=" ".join(("SQ_WAVE_CYCLES",) + SQ_CYCLES)) + "`", ""]
    return "\n".join(head + lines + [""])


def _clean_kernel_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0][-70:]


def summarize_kernel_stats(run_dir: str, command: str) -> str:
    """The --stats table of a rocprofv3 --kernel-trace run, plus per-grid averages from its trace
    (the prefill append and the one-token append are the same kernel on different grids)."""
    import csv
    with open(os.path.join(run_dir, "run_kernel_stats.csv")) as fh:
        rows = list(csv.DictReader(fh))
    out = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
           "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {_clean_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    per = {}
    with open(os.path.join(run_dir, "run_kernel_trace.csv")) as fh:
        for r in csv.DictReader(fh):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            key = (_clean_kernel_name(r["Kernel_Name"]), grid)
            per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out += ["", "Per grid (from the kernel trace):", "",
            "| kernel | grid (work-items) | calls | average us | median us |", "|---|---|---|---|---|"]
    for (k, g), d in sorted(per.items()):
        out.append(f"| {k} | {g} | {len(d)} | {np.mean(d):.2f} | {np.median(d):.2f} |")
    return "\n".join(out + [""])


def cpu_baseline(shape, k, v, slots, plan, q) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of the same workload."""
    from oracle import kvq_oracle as O
    cores = len(os.sched_getaffinity(0))
    n_seq = shape.batch if shape.batch <= 16 else 8
    n_tok = n_seq * shape.context_lens[0]
    cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
    t0 = time.perf_counter()
    O.append(cache, k[:n_tok], v[:n_tok], slots[:n_tok], shape.hadamard_block, shape.token_scale)
    t1 = time.perf_counter()
    lens = np.asarray(shape.context_lens[:n_seq])
    O.decode(cache, q[:n_seq], plan.block_table[:n_seq], lens, shape.num_kv_heads, shape.hadamard_block)
    t2 = time.perf_counter()
    ab = append_bytes(n_tok, shape.num_kv_heads, shape.bits)
    db = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
    return {
        "value": round((ab + db) / (t2 - t0) / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"append of {n_tok} prefill tokens x {shape.num_kv_heads} KV heads ({t1 - t0:.1f} s) + decode of "
                  f"{n_seq} sequences x {shape.num_q_heads} heads over {shape.context_lens[0]} tokens ({t2 - t1:.1f} s)",
        "append_GBps": round(ab / (t1 - t0) / 1e9, 4), "decode_GBps": round(db / (t2 - t1) / 1e9, 4),
        "decode_tokens_per_s": round(n_seq / (t2 - t1), 3),
    }


# ----------------------------------------------------------------------------- measured ceiling

class Ceiling:
    """Streaming probes (libkvq_stream.so) at a kernel's launch shape: how fast HBM serves a launch of
    the same grid, workgroup size and bytes that only moves bytes (16-byte non-temporal loads,
    16-byte stores, linear). Launches rotate over 1.5 GiB pools, so the 256 MB last-level cache
    cannot serve them. The paged kernels' reads are scattered page by page; the probe's linear
    stream is an upper bound for them."""
    POOL = 1536 << 20

    def __init__(self, dev):
        import torch
        from paged_decode_attention_amd import stream_probe
        self.sp = stream_probe
        self.src = torch.ones(self.POOL, dtype=torch.uint8, device=dev)
        self.dst = torch.zeros(self.POOL, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def measure(self, name, read_bytes, write_bytes, read_units, write_units, grid, block, stream, n_blocks=6,
                per_block=10, layout=0):
        """GB/s of (read + write) bytes per launch, median over blocks of ``per_block`` launches."""
        import torch
        rows = max(-(-read_bytes // (16 * read_units)) if read_units else 0,
                   -(-write_bytes // (16 * write_units)) if write_units else 0)
        rb, wb = rows * read_units * 16, rows * write_units * 16
        step_r, step_w = -(-rb // (1 << 20)) << 20, -(-wb // (1 << 20)) << 20

        def launch(i):
            so = (i * step_r) % max(1, self.POOL - rb) // 4096 * 4096 if rb else 0
            do = (i * step_w) % max(1, self.POOL - wb) // 4096 * 4096 if wb else 0
            self.sp.probe(self.src, self.dst, rows, read_units, write_units, grid, block, self.sink, stream, so, do,
                          layout=layout)
        for i in range(5):
            launch(i)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_blocks)]
        for j in range(n_blocks):
            evs[j][0].record(stream)
            for i in range(per_block):
                launch(5 + j * per_block + i)
            evs[j][1].record(stream)
        torch.cuda.synchronize()
        ms = np.array([e[0].elapsed_time(e[1]) / per_block for e in evs])
        med = float(np.median(ms))
        lay = (("reads and writes in every wave", "reader and writer workgroups")[layout]
               if read_units and write_units else "one linear stream")
        return {"pattern": name, "layout": lay,
                "GBps": round((rb + wb) / med / 1e6, 1), "read_bytes": rb, "write_bytes": wb,
                "grid": grid, "block": block, "median_us": round(med * 1e3, 2),
                "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 2),
                "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2)}

    def for_decode(self, nbytes, waves, stream):
        """A decode launch: one 64-lane workgroup per split wave, reading ``nbytes``."""
        return self.measure("read-only, non-temporal", nbytes, 0, 32, 0, waves, 64, stream)

    @staticmethod
    def append_shape(tokens, heads, bits):
        """(workgroups, threads per workgroup, read units, write units) of an append of ``tokens``
        tokens x ``heads`` KV heads: one wave per (16-token tile, KV head) item, four per 256-thread
        workgroup; per token-head 512 bytes read (bf16 K and V) and 2 (128 bits / 8) + 16 written
        (codes, scale and zero), in 16-byte units."""
        items = -(-tokens // 16) * heads
        return -(-items // 4), 256, 512 // 16, (2 * 128 * bits // 8 + 16) // 16

    def for_append(self, tokens, heads, bits, stream, patterns=("mix",)):
        """An append launch's shape moving the append's bytes (see append_shape)."""
        grid, _, rd_u, wr_u = self.append_shape(tokens, heads, bits)
        token_heads = tokens * heads
        rd, wr = 16 * rd_u, 16 * wr_u
        out = {}
        total = token_heads * (rd + wr)
        if "mix" in patterns:
            # both layouts; the faster one is the ceiling
            name = f"read/write mix {rd}:{wr} ({100 * rd / (rd + wr):.0f}/{100 * wr / (rd + wr):.0f})"
            tries = [self.measure(name, token_heads * rd, token_heads * wr, rd // 16, wr // 16, grid, 256, stream,
                                  layout=lay) for lay in (0, 1)]
            out["mix"] = max(tries, key=lambda t: t["GBps"])
            out["mix_other_layout"] = min(tries, key=lambda t: t["GBps"])
        if "read" in patterns:
            out["read"] = self.measure("read-only, non-temporal", total, 0, 32, 0, grid, 256, stream)
        if "write" in patterns:
            out["write"] = self.measure("write-only", 0, total, 0, 32, grid, 256, stream)
        if "copy" in patterns:
            tries = [self.measure("copy (half read, half written)", total // 2, total // 2, 16, 16, grid, 256, stream,
                                  layout=lay) for lay in (0, 1)]
            out["copy"] = max(tries, key=lambda t: t["GBps"])
        return out


def _decode_waves(batch, num_q_heads, num_kv_heads, max_len, page_size):
    """Waves of the one-query decode launch: splits (read back from the workspace size, which holds
    a (128 + 2)-float row per split, sequence and query head) times sequences times KV heads."""
    from paged_decode_attention_amd import kvq
    w = kvq.decode_workspace_size(batch, num_q_heads, num_kv_heads, max_len, page_size)
    splits = round(w / (batch * num_q_heads * (128 * 4 + 8))) if w else 1
    return splits * batch * num_kv_heads


def _pcts(ms):
    ms = np.asarray(ms)
    return {"median_ms": round(float(np.median(ms)), 5), "p10_ms": round(float(np.percentile(ms, 10)), 5),
            "p90_ms": round(float(np.percentile(ms, 90)), 5)}


def _roofline(kernel, nbytes, ms, ceiling_gbps, traffic):
    gb = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gb, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gb / PEAK_HBM_GBPS, 4),
            "frac_of_measured_ceiling": round(gb / ceiling_gbps, 4) if ceiling_gbps else None,
            "measured_ceiling": ceiling_gbps, "traffic": traffic, "kernel": kernel, "bytes_per_launch": nbytes}


def _say(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _chunk_attention_rates(lens, qlen, num_q_heads, ms):
    """Rates of a several-query attention call: the algorithmic QK + PV multiply-adds over every
    query's causal window, and - for the large-chunk kernel - the fp16 matrix-core work it runs
    (three passes per score: QK with the query's hi and lo parts, then PV, over whole 64-token
    tiles) against the dense fp16 peak."""
    causal = float(np.sum([qlen * (int(n) - qlen) + qlen * (qlen + 1) / 2 for n in lens]))
    flops = 4.0 * 128 * num_q_heads * causal
    tiles = float(np.sum([np.ceil(int(n) / 64.0) for n in lens]))
    mfma_flops = 3 * 2.0 * 128 * 64 * tiles * qlen * num_q_heads
    return {"attention_TFLOPs": round(flops / ms / 1e9, 2), "mfma_fp16_TFLOPs": round(mfma_flops / ms / 1e9, 1),
            "mfma_frac_of_fp16_dense_peak": round(mfma_flops / ms / 1e9 / PEAK_FP16_TFLOPS, 3)}


def _block_times(fn, n_blocks, per_block, stream, start=0):
    """Per-call ms of fn over n_blocks event-bracketed blocks of per_block back-to-back calls."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_blocks)]
    for j in range(n_blocks):
        evs[j][0].record(stream)
        for i in range(per_block):
            fn(start + j * per_block + i)
        evs[j][1].record(stream)
    torch.cuda.synchronize()
    return np.array([e[0].elapsed_time(e[1]) / per_block for e in evs])


def record_llama2_70b(dev, stream, ceiling):
    """The Llama-2-70B-shaped step: 80 independent layer caches (4 x 32768 tokens, 64/8 heads, INT4);
    per layer one fused decode step (append of each sequence's new token + attention over 32769
    tokens + split merge). Returns the record and the layer-0 decode-step closures' inputs."""
    from paged_decode_attention_amd import workloads as W
    shape = W.config("llama2_70b")
    layers = []
    for l in range(shape.layers):
        plan = W.plan_pages(shape, extra_tokens=1, layer=l)
        caches = _filled_caches(shape, plan, 1, dev, stream, layer=l)
        layers.append(_decode_step_fns(shape, plan, caches, dev, stream, layer=l))
    _say(f"{shape.name}: {shape.layers} layer caches filled")

    def step(i):
        for append, _, _ in layers:
            append.fused(0)

    def attention(i):
        for _, attend, _ in layers:
            attend(0)
    for i in range(3):
        step(i)
        attention(i)
    torch_sync()
    steps = _block_times(step, 8, 1, stream)
    att = _block_times(attention, 4, 1, stream)
    lens = layers[0][2]
    b_att = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
    b_app = append_bytes(shape.batch, shape.num_kv_heads, shape.bits)
    per_layer = steps / shape.layers
    t_layer = float(np.mean(per_layer))
    waves = _decode_waves(shape.batch, shape.num_q_heads, shape.num_kv_heads, int(np.max(lens)), shape.page_size)
    del layers, step, attention
    torch_empty_cache()
    ceil = ceiling.for_decode(b_att, waves, stream)
    t_dec = [stored_traffic(shape.name, k) for k in ("decode_mfma_kernel", "decode_merge_splits_kernel")]
    t_dec = None if None in t_dec else sum(t_dec)
    step_ms = float(np.mean(steps))
    rec = {
        "workload": "llama2_70b: 4 seq x 32768 tokens, 64/8 heads, head_dim 128, page 16, Hadamard block 128, INT4, "
                    "80 independent layer caches; one step = per layer a fused decode step (append of the new token "
                    "+ attention over 32769 tokens + split merge)",
        "layers": shape.layers, "step_ms": round(step_ms, 4), "step": _pcts(steps),
        "tokens_per_s": round(shape.batch / (step_ms * 1e-3), 1),
        "step_GBps": round((b_att + b_app) * shape.layers / (step_ms * 1e-3) / 1e9, 1),
        "decode_step_per_layer_ms": round(t_layer, 5),
        "attention_only_per_layer_ms": round(float(np.mean(att)) / shape.layers, 5),
        "roofline": _roofline("kvq_decode_step, one layer (decode + split merge launches)", b_att + b_app, t_layer,
                              ceil["GBps"], t_dec),
        "ceiling_decode_shape": ceil,
    }
    return rec


def record_oscar(dev, stream, ceiling):
    """The OScaR INT2 shape (32 x 16384 tokens, 28/4 heads, rotation + per-token scaling + INT2):
    512-token chunk appends that land mid-page, then decode attention over 16385 tokens."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    shape = W.config("oscar_int2")
    plan = W.plan_pages(shape, extra_tokens=1)
    calls = W.chunk_schedule(shape)
    n_tok = sum(len(sq) for sq, _ in calls)
    k, v = W.draw_kv_device(shape, n_tok, dev)
    cache = kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
    slot_list, offs, o = [], [], 0
    for sq, ps in calls:
        slot_list.append(torch.from_numpy(W.slots_for_positions(plan, shape.page_size, sq, ps)).to(dev))
        offs.append((o, o + len(sq)))
        o += len(sq)
    full = [i for i, (a, b) in enumerate(offs) if b - a == shape.batch * shape.chunk]
    for i, ((a, b), sl) in enumerate(zip(offs, slot_list)):
        if i not in full:
            kvq.rotate_quantize_append(k[a:b], v[a:b], sl, cache, shape.hadamard_block, shape.token_scale,
                                       stream=stream)

    def chunk(i):
        (a, b), sl = offs[full[i % len(full)]], slot_list[full[i % len(full)]]
        kvq.rotate_quantize_append(k[a:b], v[a:b], sl, cache, shape.hadamard_block, shape.token_scale, stream=stream)
    # the chunks in order, each timed on its own (one event pair per chunk): the serving loop's calls
    chunk_ms = _block_times(chunk, len(full), 1, stream)
    del k, v
    # the attention of the last 512-token chunk over its sequence (16384 tokens): the large-chunk kernel
    lens_c = np.asarray(shape.context_lens, dtype=np.int32)
    gq = torch.Generator(device=dev)
    gq.manual_seed(shape.seed + shape.chunk)
    qc = torch.randn((shape.batch, shape.chunk, shape.num_q_heads, 128), generator=gq, device=dev).to(torch.bfloat16)
    qlc = torch.full((shape.batch,), shape.chunk, dtype=torch.int32, device=dev)
    btc, lens_cd = torch.from_numpy(plan.block_table).to(dev), torch.from_numpy(lens_c).to(dev)
    outc = torch.empty((shape.batch, shape.chunk, shape.num_q_heads, 128), dtype=torch.float32, device=dev)

    def chunk_attention(i):
        kvq.paged_prefill_attention(qc, qlc, cache, btc, lens_cd, int(lens_c.max()), shape.hadamard_block, out=outc,
                                    stream=stream)
    chunk_attention(0)
    ca_ms = _block_times(chunk_attention, 3, 2, stream)
    ca_kernel = kvq.prefill_kernel(shape.batch, shape.chunk, shape.num_q_heads, shape.num_kv_heads)
    del qc, outc
    copies = [cache] + [kvq.PagedKVCache(cache.k_codes.clone(), cache.v_codes.clone(), cache.k_sz.clone(),
                                         cache.v_sz.clone(), cache.bits) for _ in range(7)]
    append, attend, lens = _decode_step_fns(shape, plan, copies, dev, stream)
    for i in range(5):
        attend(i)
        append.fused(i)
    att = _block_times(attend, 6, 10, stream)
    fused = _block_times(append.fused, 6, 10, stream)
    b_att = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
    b_chunk = append_bytes(shape.batch * shape.chunk, shape.num_kv_heads, shape.bits)
    b_app = append_bytes(shape.batch, shape.num_kv_heads, shape.bits)
    waves = _decode_waves(shape.batch, shape.num_q_heads, shape.num_kv_heads, int(np.max(lens)), shape.page_size)
    del copies, cache, append, attend
    torch_empty_cache()
    t_bf, gb_bf = _bf16_attention(shape, plan, dev, stream)
    torch_empty_cache()
    c_dec = ceiling.for_decode(b_att, waves, stream)
    c_app = ceiling.for_append(shape.batch * shape.chunk, shape.num_kv_heads, shape.bits, stream)["mix"]
    t_dec = [stored_traffic(shape.name, kk) for kk in ("decode_mfma_kernel", "decode_merge_splits_kernel")]
    t_dec = None if None in t_dec else sum(t_dec)
    t_ms = float(np.mean(att))
    c_ms = float(np.mean(chunk_ms))
    f_ms = float(np.mean(fused))
    return {
        "workload": "oscar_int2: 32 seq x 16384 tokens, 28/4 heads, head_dim 128, page 16, Hadamard block 128, "
                    "per-token scaling, INT2; 512-token chunk appends landing mid-page, then decode attention over "
                    "16385 tokens",
        "attention": _pcts(att), "decode_tokens_per_s": round(shape.batch / (t_ms * 1e-3), 1),
        "fused_decode_step": _pcts(fused), "fused_tokens_per_s": round(shape.batch / (f_ms * 1e-3), 1),
        "fused_decode_step_GBps": round((b_att + b_app) / (f_ms * 1e-3) / 1e9, 1),
        "chunk_append": dict(_pcts(chunk_ms), chunks=len(full), bytes=b_chunk,
                             tokens_per_s=round(shape.batch * shape.chunk / (c_ms * 1e-3), 1)),
        "chunk_attention": dict(_pcts(ca_ms), queries_per_seq=shape.chunk,
                                kernel="large-chunk" if ca_kernel == 1 else "split",
                                query_tokens_per_s=round(shape.batch * shape.chunk / (float(np.mean(ca_ms)) * 1e-3), 1),
                                **_chunk_attention_rates(lens_c, shape.chunk, shape.num_q_heads,
                                                         float(np.mean(ca_ms)))),
        "roofline": _roofline("kvq_paged_decode_attention (decode + split merge launches)", b_att, t_ms,
                              c_dec["GBps"], t_dec),
        "roofline_chunk_append": _roofline("kvq_rotate_quantize_append, 32 x 512-token chunk", b_chunk, c_ms,
                                           c_app["GBps"], stored_traffic(shape.name, "append_kernel")),
        "ceiling_decode_shape": c_dec, "ceiling_chunk_append_shape": c_app,
        "baseline_bf16_decode": {"avg_ms": round(t_bf, 5), "GBps": round(gb_bf, 1),
                                 "speedup_of_int2_decode": round(t_bf / t_ms, 2),
                                 "cache_bytes_ratio": round(512 / (2 * 128 * shape.bits // 8 + 16), 2)},
    }


def record_sweep(dev, stream):
    """The concurrency sweep on the Llama-3-8B layer shape: batch 1 ... 256, ragged contexts
    U{512..8192}, Hadamard block 64; one fused decode step (append + attention) per batch size."""
    from paged_decode_attention_amd import workloads as W
    rows = []
    for b in (1, 8, 32, 128, 256):
        shape = W.config(f"sweep_b{b}")
        plan = W.plan_pages(shape, extra_tokens=1)
        n_copies = int(min(32, max(1, math.ceil(1.1e9 / _cache_bytes(shape, plan.num_pages)))))
        caches = _filled_caches(shape, plan, n_copies, dev, stream)
        append, attend, lens = _decode_step_fns(shape, plan, caches, dev, stream)
        for i in range(5):
            append.fused(i)
            attend(i)
        fused = _block_times(append.fused, 5, 10, stream)
        att = _block_times(attend, 5, 10, stream)
        b_att = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
        b_app = append_bytes(shape.batch, shape.num_kv_heads, shape.bits)
        f_ms, a_ms = float(np.mean(fused)), float(np.mean(att))
        rows.append({"batch": b, "tokens": int(np.sum(lens)), "fused_decode_step": _pcts(fused),
                     "tokens_per_s": round(b / (f_ms * 1e-3), 1),
                     "fused_GBps": round((b_att + b_app) / (f_ms * 1e-3) / 1e9, 1),
                     "attention": _pcts(att), "attention_GBps": round(b_att / (a_ms * 1e-3) / 1e9, 1)})
        del caches, append, attend
        torch_empty_cache()
    return {"workload": "sweep: Llama-3-8B layer shape, batch 1/8/32/128/256, ragged contexts U{512..8192}, page 16, "
                        "Hadamard block 64, INT4; one fused decode step per batch (eager launches)",
            "rows": rows}


def record_tiny(dev, stream):
    """The tiny single-layer check (1 x 512 tokens, 8/8 heads, Hadamard block 32): latency of the
    prefill append and of the fused decode step, eager launches."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    shape = W.config("tiny")
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    slots = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, seq, pos)).to(dev)
    k, v = W.draw_kv_device(shape, len(seq), dev)
    cache = kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
    pre = _block_times(lambda i: kvq.rotate_quantize_append(k, v, slots, cache, shape.hadamard_block, 0,
                                                            stream=stream), 5, 10, stream)
    append, _, _ = _decode_step_fns(shape, plan, [cache], dev, stream)
    fused = _block_times(append.fused, 5, 10, stream)
    return {"workload": "tiny: 1 seq x 512 tokens, 8/8 heads, head_dim 128, page 16, Hadamard block 32, INT4",
            "prefill_append": _pcts(pre), "fused_decode_step": _pcts(fused)}


def cpu_decode_baseline(name, n_seq, extrapolate=1.0, note=""):
    """The oracle (as it stands) on the first n_seq sequences of a workload: its append of their
    prefill (set-up, timed separately) and its decode (one query per head) over the prefill; GB/s of
    the decode's algorithmic bytes, and tokens/s of the decode scaled to the whole workload by
    ``extrapolate`` (the sample's share of it)."""
    from oracle import kvq_oracle as O
    from paged_decode_attention_amd import workloads as W
    shape = W.config(name)
    s = shape.with_(batch=n_seq, context_lens=tuple(shape.context_lens[:n_seq]))
    plan = W.plan_pages(s, extra_tokens=0)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.bits)
    t0 = time.perf_counter()
    O.append(cache, k, v, W.slots_for_positions(plan, s.page_size, seq, pos), s.hadamard_block, s.token_scale)
    t1 = time.perf_counter()
    q = W.draw_q(s)
    O.decode(cache, q, plan.block_table, np.asarray(s.context_lens), s.num_kv_heads, s.hadamard_block)
    t2 = time.perf_counter()
    nb = decode_bytes(np.asarray(s.context_lens), s.num_q_heads, s.num_kv_heads, s.bits, s.page_size)
    ab = append_bytes(len(seq), s.num_kv_heads, s.bits)
    out = {"kind": "oracle", "cores": len(os.sched_getaffinity(0)),
           "sample": f"{name}: append of the prefill of {n_seq} of {shape.batch} sequences ({len(seq)} tokens, "
                     f"{t1 - t0:.1f} s), then decode of those {n_seq} x {s.num_q_heads} heads ({t2 - t1:.1f} s)" + note,
           "decode_GBps": round(nb / (t2 - t1) / 1e9, 5), "append_GBps": round(ab / (t1 - t0) / 1e9, 5),
           "decode_s": round(t2 - t1, 3)}
    if extrapolate != 1.0:
        out["extrapolated"] = True
        out["extrapolated_decode_step_s"] = round((t2 - t1) * extrapolate, 2)
        out["decode_tokens_per_s"] = round(shape.batch / ((t2 - t1) * extrapolate), 5)
    else:
        out["decode_tokens_per_s"] = round(shape.batch / (t2 - t1), 5)
    return out


def counters_other(args, dev):
    """--counters for the Llama-2-70B and OScaR workloads: set-up, three calibration copies of known
    size, then the dispatches the counters are read on (no copy after the calibration)."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    stream = torch.cuda.current_stream()
    shape = W.config(args.workload)
    if shape.name == "llama2_70b":
        layers = []
        for l in range(4):
            plan = W.plan_pages(shape, extra_tokens=1, layer=l)
            caches = _filled_caches(shape, plan, 1, dev, stream, layer=l)
            layers.append(_decode_step_fns(shape, plan, caches, dev, stream, layer=l))

        def run():
            for i in range(args.steps):
                for append, _, _ in layers:
                    append.fused(0)
        what = f"{args.steps} x 4 layers of fused decode steps"
    else:
        plan = W.plan_pages(shape, extra_tokens=1)
        calls = W.chunk_schedule(shape)
        n_tok = sum(len(sq) for sq, _ in calls)
        k, v = W.draw_kv_device(shape, n_tok, dev)
        cache = kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
        work, o = [], 0
        for sq, ps in calls:
            sl = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, sq, ps)).to(dev)
            work.append((o, o + len(sq), sl))
            o += len(sq)
        full = [w for w in work if w[1] - w[0] == shape.batch * shape.chunk]
        for a, b, sl in work:
            if b - a != shape.batch * shape.chunk:
                kvq.rotate_quantize_append(k[a:b], v[a:b], sl, cache, shape.hadamard_block, shape.token_scale,
                                           stream=stream)
        copies = [kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
                  for _ in range(4)]
        _, attend, _ = _decode_step_fns(shape, plan, copies, dev, stream)
        # a 512-token chunk's attention over 16384 tokens per sequence (the large-chunk kernel)
        lens_c = torch.from_numpy(np.asarray(shape.context_lens, dtype=np.int32)).to(dev)
        qc = torch.randn((shape.batch, shape.chunk, shape.num_q_heads, 128), device=dev).to(torch.bfloat16)
        qlc = torch.full((shape.batch,), shape.chunk, dtype=torch.int32, device=dev)
        btc = torch.from_numpy(plan.block_table).to(dev)

        def run():
            for a, b, sl in full[:args.steps]:
                kvq.rotate_quantize_append(k[a:b], v[a:b], sl, cache, shape.hadamard_block, shape.token_scale,
                                           stream=stream)
            for i in range(args.steps):
                attend(i)
            for i in range(2):
                kvq.paged_prefill_attention(qc, qlc, cache, btc, lens_c, max(shape.context_lens), shape.hadamard_block,
                                            stream=stream)
        what = (f"{min(args.steps, len(full))} chunk appends of 32 x 512 tokens, then {args.steps} decodes and "
                f"2 attentions of a 512-token chunk")
    torch.cuda.synchronize()
    src = torch.ones(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    run()
    torch.cuda.synchronize()
    print(f"counters run ({shape.name}): 3 calibration copies of {CALIBRATION_BYTES} bytes, {what}", flush=True)


def torch_sync():
    import torch
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- workload suite

def _cache_bytes(shape, num_pages) -> int:
    return num_pages * shape.num_kv_heads * shape.page_size * (2 * 128 * shape.bits // 8 + 16)


def _timed(fn, n, stream):
    """Average ms of fn(i) over n back-to-back calls (events on the launch stream)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _filled_caches(shape, plan, n_copies, dev, stream, layer=0):
    """n_copies caches holding the whole prefill of ``shape`` (device-drawn inputs)."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    seq, pos = W.prefill_order(shape)
    slots = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, seq, pos)).to(dev)
    k, v = W.draw_kv_device(shape, len(seq), dev, layer=layer)
    caches = []
    for _ in range(n_copies):
        c = kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
        kvq.rotate_quantize_append(k, v, slots, c, shape.hadamard_block, shape.token_scale, stream=stream)
        caches.append(c)
    del k, v
    torch.cuda.synchronize()
    return caches


def _timed_graph(fn, n_inner, n_rep):
    """Average ms of fn(i) when n_inner calls are captured in one HIP graph and the graph is replayed
    n_rep times: the GPU time of launch-bound calls without the host's per-call launch cost. fn must
    launch on the current stream (the capture stream while capturing)."""
    import torch
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_inner):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_rep):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (n_rep * n_inner)


def _decode_step_fns(shape, plan, caches, dev, stream, layer=0):
    """(append, attend) closures for one decode step of ``shape`` on cache copy i (stream None: the
    current stream at call time)."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    dseq, dpos = W.decode_positions(shape)
    dslots = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, dseq, dpos)).to(dev)
    kn, vn = W.draw_kv_device(shape, shape.batch, dev, layer=layer, stream="decode")
    q = W.draw_q_device(shape, dev, layer=layer)
    lens = np.asarray(shape.context_lens, dtype=np.int32) + 1
    lens_d = torch.from_numpy(lens).to(dev)
    bt = torch.from_numpy(plan.block_table).to(dev)
    max_len = int(lens.max())
    ws = kvq.decode_workspace(kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len,
                                                        shape.page_size), dev)
    out = torch.empty((shape.batch, shape.num_q_heads, 128), dtype=torch.float32, device=dev)

    def append(i):
        kvq.rotate_quantize_append(kn, vn, dslots, caches[i % len(caches)], shape.hadamard_block, shape.token_scale,
                                   stream=stream)

    def attend(i):
        kvq.paged_decode_attention(q, caches[i % len(caches)], bt, lens_d, max_len, shape.hadamard_block, out=out,
                                   workspace=ws, stream=stream)

    def fused(i):
        kvq.decode_step(q, kn, vn, caches[i % len(caches)], bt, lens_d, max_len, shape.hadamard_block,
                        token_scale=shape.token_scale, out=out, workspace=ws, stream=stream)
    append.fused = fused
    return append, attend, lens


def _bf16_attention(shape, plan, dev, stream, n_copies=None, layer=0):
    """Average ms (and GB/s) of the bf16 baseline decode over caches holding the same synthetic
    sequences as the low-bit run: the prefill plus the decode step's new token."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    cache_bytes = plan.num_pages * shape.num_kv_heads * shape.page_size * 128 * 2 * 2
    if n_copies is None:
        n_copies = int(min(16, max(1, math.ceil(1.1e9 / cache_bytes))))
    seq, pos = W.prefill_order(shape)
    slots = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, seq, pos)).to(dev)
    k, v = W.draw_kv_device(shape, len(seq), dev, layer=layer)
    dseq, dpos = W.decode_positions(shape)
    dslots = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, dseq, dpos)).to(dev)
    kn, vn = W.draw_kv_device(shape, shape.batch, dev, layer=layer, stream="decode")
    lens = np.asarray(shape.context_lens, dtype=np.int64) + 1
    caches = []
    for _ in range(n_copies):
        c = kvq.PagedKVCacheBF16.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, device=dev)
        kvq.bf16_cache_write(k, v, slots, c, stream=stream)
        kvq.bf16_cache_write(kn, vn, dslots, c, stream=stream)
        caches.append(c)
    del k, v
    q = W.draw_q_device(shape, dev, layer=layer)
    lens_d = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev)
    bt = torch.from_numpy(plan.block_table).to(dev)
    max_len = int(np.max(lens))
    ws = kvq.decode_workspace(kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len,
                                                        shape.page_size), dev)
    out = torch.empty((shape.batch, shape.num_q_heads, 128), dtype=torch.float32, device=dev)

    def attend(i):
        kvq.paged_decode_attention_bf16(q, caches[i % n_copies], bt, lens_d, max_len, out=out, workspace=ws,
                                        stream=stream)
    for i in range(5):
        attend(i)
    ms = _timed(attend, 50, stream)
    toks = int(np.sum(lens))
    nbytes = toks * shape.num_kv_heads * 512 + shape.batch * shape.num_q_heads * 128 * 6
    del caches
    return ms, nbytes / ms / 1e6


def _line(**kw):
    return kw


def suite_sweep(dev, stream, cpu):
    from paged_decode_attention_amd import workloads as W
    rows = []
    for b in (1, 8, 32, 128, 256):
        for hb in (64, 1):
            shape = W.config(f"sweep_b{b}", hadamard_block=hb)
            plan = W.plan_pages(shape, extra_tokens=1)
            n_copies = int(min(32, max(1, math.ceil(1.1e9 / _cache_bytes(shape, plan.num_pages)))))
            caches = _filled_caches(shape, plan, n_copies, dev, stream)
            append, attend, lens = _decode_step_fns(shape, plan, caches, dev, stream)
            for i in range(5):
                append(i), attend(i)
            n = 60
            t_app = _timed(append, n, stream)
            t_att = _timed(attend, n, stream)
            t_step = _timed(lambda i: (append(i), attend(i)), n, stream)
            b_att = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
            b_app = append_bytes(shape.batch, shape.num_kv_heads, shape.bits)
            rows.append(_line(workload=f"sweep batch {b}, Hadamard block {hb}" + (" (plain INT4)" if hb == 1 else ""),
                              batch=b, hadamard_block=hb, cache_copies=n_copies, step_ms=round(t_step, 5),
                              append_ms=round(t_app, 5), attention_ms=round(t_att, 5),
                              attention_GBps=round(b_att / t_att / 1e6, 1),
                              step_GBps=round((b_att + b_app) / t_step / 1e6, 1),
                              tokens_per_s=round(b / (t_step * 1e-3), 1)))
            if b <= 32:
                # small batches are launch-bound: the same calls replayed from a HIP graph
                g_append, g_attend, _ = _decode_step_fns(shape, plan, caches, dev, None)
                t_g_att = _timed_graph(g_attend, 20, 10)
                t_g_step = _timed_graph(lambda i: (g_append(i), g_attend(i)), 20, 10)
                rows[-1].update(graph_attention_ms=round(t_g_att, 5), graph_step_ms=round(t_g_step, 5),
                                graph_attention_GBps=round(b_att / t_g_att / 1e6, 1),
                                graph_tokens_per_s=round(b / (t_g_step * 1e-3), 1))
            del caches
            if hb == 64:
                t_bf, gb_bf = _bf16_attention(shape, plan, dev, stream)
                rows[-1].update(bf16_attention_ms=round(t_bf, 5), bf16_attention_GBps=round(gb_bf, 1),
                                attention_speedup_vs_bf16=round(t_bf / t_att, 2),
                                cache_bytes_ratio_bf16=round(512 / (2 * 128 * shape.bits // 8 + 16), 2))
            if cpu and hb == 64 and b <= 8:
                rows[-1]["cpu_oracle"] = _cpu_decode_sample(shape, n_seq=min(b, 2))
    return rows


def suite_llama2_70b(dev, stream, cpu):
    """80 independent per-layer caches; one step = per layer, append one token per sequence and
    attend (a new query per layer)."""
    from paged_decode_attention_amd import workloads as W
    shape = W.config("llama2_70b")
    layers = []
    for l in range(shape.layers):
        plan = W.plan_pages(shape, extra_tokens=1, layer=l)
        caches = _filled_caches(shape, plan, 1, dev, stream, layer=l)
        layers.append(_decode_step_fns(shape, plan, caches, dev, stream, layer=l))
        if l % 20 == 19:
            print(f"llama2_70b: {l + 1} layer caches filled", file=sys.stderr, flush=True)

    def step(i):
        for append, attend, _ in layers:
            append(0)
            attend(0)

    def attention_only(i):
        for _, attend, _ in layers:
            attend(0)

    def step_fused(i):
        for append, _, _ in layers:
            append.fused(0)
    for i in range(2):
        step(i)
        step_fused(i)
    t_step = _timed(step, 10, stream)
    t_att = _timed(attention_only, 10, stream)
    t_fused = _timed(step_fused, 10, stream)
    lens = layers[0][2]
    b_att = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size) * shape.layers
    b_app = append_bytes(shape.batch, shape.num_kv_heads, shape.bits) * shape.layers
    row = _line(workload="Llama-2-70B shape, 4 x 32768 tokens, 64/8 heads, 80 layers (one step)", batch=shape.batch,
                layers=shape.layers, step_ms=round(t_step, 4), fused_step_ms=round(t_fused, 4),
                fused_tokens_per_s=round(shape.batch / (t_fused * 1e-3), 1), attention_ms_80_layers=round(t_att, 4),
                attention_ms_per_layer=round(t_att / shape.layers, 5), attention_GBps=round(b_att / t_att / 1e6, 1),
                step_GBps=round((b_att + b_app) / t_step / 1e6, 1),
                tokens_per_s=round(shape.batch / (t_step * 1e-3), 1))
    del layers, step, attention_only, step_fused
    torch_empty_cache()
    plan0 = W.plan_pages(shape, extra_tokens=1)
    t_bf, gb_bf = _bf16_attention(shape, plan0, dev, stream, n_copies=4)
    row.update(bf16_attention_ms_per_layer=round(t_bf, 5), bf16_attention_GBps=round(gb_bf, 1),
               attention_speedup_vs_bf16=round(t_bf / (t_att / shape.layers), 2),
               cache_bytes_ratio_bf16=round(512 / (2 * 128 * shape.bits // 8 + 16), 2))
    if cpu:
        c = _cpu_decode_sample(shape, n_seq=1)
        c["extrapolated_step_s"] = round(c["seconds_per_seq"] * shape.batch * shape.layers, 1)
        row["cpu_oracle"] = c
    return [row]


def suite_oscar(dev, stream, cpu):
    """Chunked prefill (first 1..15 tokens, then 512-token chunks that start mid-page), then a decode step."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    shape = W.config("oscar_int2")
    plan = W.plan_pages(shape, extra_tokens=1)
    calls = W.chunk_schedule(shape)
    n_tok = sum(len(s) for s, _ in calls)
    k, v = W.draw_kv_device(shape, n_tok, dev)
    cache = kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
    slot_list, offs, o = [], [], 0
    for sq, ps in calls:
        slot_list.append(torch.from_numpy(W.slots_for_positions(plan, shape.page_size, sq, ps)).to(dev))
        offs.append((o, o + len(sq)))
        o += len(sq)
    torch.cuda.synchronize()
    # the short first chunks (1..15 tokens per sequence), then the 512-token chunks back to back as a
    # serving loop issues them (each lands mid-page), timed together
    full_calls = [i for i, (a, b) in enumerate(offs) if b - a == shape.batch * shape.chunk]
    for i, ((a, b), sl) in enumerate(zip(offs, slot_list)):
        if i not in full_calls:
            kvq.rotate_quantize_append(k[a:b], v[a:b], sl, cache, shape.hadamard_block, shape.token_scale,
                                       stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in full_calls:
        (a, b), sl = offs[i], slot_list[i]
        kvq.rotate_quantize_append(k[a:b], v[a:b], sl, cache, shape.hadamard_block, shape.token_scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    chunk_mean_ms = e0.elapsed_time(e1) / max(1, len(full_calls))
    del k, v
    # attention cycles over 8 copies (1.3 GB) so that the 256 MB last-level cache cannot serve it
    copies = [cache] + [kvq.PagedKVCache(cache.k_codes.clone(), cache.v_codes.clone(), cache.k_sz.clone(),
                                         cache.v_sz.clone(), cache.bits) for _ in range(7)]
    append, attend, lens = _decode_step_fns(shape, plan, copies, dev, stream)
    for i in range(5):
        attend(i)
    t_att = _timed(attend, 50, stream)
    t_app = _timed(append, 50, stream)
    b_att = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
    b_chunk = append_bytes(shape.batch * shape.chunk, shape.num_kv_heads, shape.bits)
    del copies, cache
    torch_empty_cache()
    t_bf, gb_bf = _bf16_attention(shape, plan, dev, stream)
    row = _line(workload="OScaR INT2 shape, 32 x 16384 tokens, 28/4 heads, chunked prefill of 512 tokens",
                bf16_attention_ms=round(t_bf, 5), bf16_attention_GBps=round(gb_bf, 1),
                attention_speedup_vs_bf16=round(t_bf / t_att, 2),
                cache_bytes_ratio_bf16=round(512 / (2 * 128 * shape.bits // 8 + 16), 2),
                batch=shape.batch, chunk_appends=len(full_calls), chunk_append_ms_mean=round(chunk_mean_ms, 5),
                chunk_append_GBps=round(b_chunk / chunk_mean_ms / 1e6, 1), attention_ms=round(t_att, 5),
                attention_GBps=round(b_att / t_att / 1e6, 1), decode_token_append_ms=round(t_app, 5),
                tokens_per_s=round(shape.batch / ((t_att + t_app) * 1e-3), 1))
    if cpu:
        row["cpu_oracle"] = _cpu_decode_sample(shape, n_seq=1)
    return [row]


def pc_write_bytes(tokens: int, heads: int, bits: int, page_size: int, d: int = 128) -> int:
    """Algorithmic bytes of kvq_pc_write_pages: bf16 K+V read; codes, a float32 scale per token and
    a float32 (scale, zero) per channel per page written for K and V; the page ids."""
    pages = tokens // page_size
    return tokens * heads * (2 * d * 2 + 2 * d * bits // 8 + 2 * 4) + pages * heads * 2 * 2 * d * 4 + pages * 4


def pc_decode_bytes(lens, num_q_heads: int, num_kv_heads: int, bits: int, page_size: int, d: int = 128) -> int:
    """Algorithmic bytes of kvq_pc_decode_attention: codes and token scales of every token in a
    complete page, each page's K and V (scale, zero) per channel, the bf16 tail tokens, block-table
    entries, bf16 q, fp32 out, the context lengths."""
    lens = np.asarray(lens)
    full = lens // page_size
    toks = int(np.sum(full)) * page_size
    tail = int(np.sum(lens - full * page_size))
    b = len(lens)
    return (toks * num_kv_heads * (2 * d * bits // 8 + 2 * 4) + int(np.sum(full)) * num_kv_heads * 2 * 2 * d * 4
            + tail * num_kv_heads * 2 * d * 2 + int(np.sum(full)) * 4 + b * num_q_heads * d * (2 + 4) + b * 4)


def suite_pc(dev, stream, cpu):
    """Per-channel OScaR pages on the OScaR INT2 shape (32 x 16384 tokens, 28/4 heads) with pages of 64
    and of 128 tokens: the whole prefill written page by page, then a decode step whose newest token
    sits in the bf16 residual window."""
    return [_pc_row(dev, stream, ps) for ps in (64, 128)]


def _pc_row(dev, stream, ps):
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    shape = W.config("oscar_int2")
    hb, bits = shape.hadamard_block, shape.bits
    bsz, heads = shape.batch, shape.num_kv_heads
    per_seq = shape.context_lens[0] // ps
    n_pages = bsz * per_seq
    k, v = W.draw_kv_device(shape, n_pages * ps, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(shape.seed + 64)
    ids = torch.randperm(n_pages, generator=g, device=dev).to(torch.int32)
    bt = ids.view(bsz, per_seq).contiguous()
    cache = kvq.PagedKVCachePC.empty(n_pages, heads, ps, bits, device=dev)
    kvq.pc_write_pages(k, v, ids, cache, hb, stream=stream)
    torch.cuda.synchronize()
    t_write = _timed(lambda i: kvq.pc_write_pages(k, v, ids, cache, hb, stream=stream), 5, stream)
    del k, v
    copies = [cache] + [kvq.PagedKVCachePC(cache.k_codes.clone(), cache.v_codes.clone(), cache.k_s.clone(),
                                           cache.v_s.clone(), cache.k_cp.clone(), cache.v_cp.clone(), bits)
                        for _ in range(7)]
    tail_k, tail_v = (torch.randn((bsz, ps, heads, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(2))
    lens_np = np.full(bsz, per_seq * ps + 1, dtype=np.int32)   # the prefill plus the new token, in the tail
    lens = torch.from_numpy(lens_np).to(dev)
    q = torch.randn((bsz, shape.num_q_heads, 128), generator=g, device=dev).to(torch.bfloat16)
    max_len = int(lens_np.max())
    ws = kvq.decode_workspace(kvq.pc_decode_workspace_size(bsz, shape.num_q_heads, heads, max_len, ps), dev)
    out = torch.empty((bsz, shape.num_q_heads, 128), dtype=torch.float32, device=dev)

    def attend(i):
        kvq.pc_decode_attention(q, copies[i % len(copies)], bt, lens, max_len, tail_k, tail_v, hb, out=out,
                                workspace=ws, stream=stream)
    for i in range(5):
        attend(i)
    t_att = _timed(attend, 50, stream)
    b_att = pc_decode_bytes(lens_np, shape.num_q_heads, heads, bits, ps)
    b_write = pc_write_bytes(n_pages * ps, heads, bits, ps)
    del copies, cache
    torch_empty_cache()
    gbps_att = b_att / t_att / 1e6
    row = _line(workload=f"OScaR per-channel INT2 pages of {ps} tokens, 32 x 16385 tokens, 28/4 heads",
                batch=bsz, page_size=ps, pages=n_pages,
                write_ms=round(t_write, 5), write_GBps=round(b_write / t_write / 1e6, 1),
                write_tokens_per_s=round(n_pages * ps / (t_write * 1e-3), 1),
                attention_ms=round(t_att, 5), attention_bytes=b_att, attention_GBps=round(gbps_att, 1),
                attention_frac_of_peak=round(gbps_att / PEAK_HBM_GBPS, 4),
                cache_bytes_per_token_head=round((2 * 128 * bits // 8 + 8) + 2 * 2 * 128 * 4 / ps, 1))
    return row


def suite_multi_query(dev, stream, cpu):
    """Several queries per sequence over the low-bit cache: speculative verification (4 draft
    tokens per sequence, Llama-3-8B shape) and a 512-token chunk of chunked prefill (OScaR INT2
    shape: the chunk's attention over its sequence so far)."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    rows = []
    for name, qlen in (("llama3_8b", 4), ("oscar_int2", 512)):
        shape = W.config(name)
        plan = W.plan_pages(shape, extra_tokens=1)
        caches = _filled_caches(shape, plan, 4, dev, stream)
        lens = np.asarray(shape.context_lens, dtype=np.int32)  # the last qlen tokens are the queries
        g = torch.Generator(device=dev)
        g.manual_seed(shape.seed + qlen)
        q = torch.randn((shape.batch, qlen, shape.num_q_heads, 128), generator=g, device=dev).to(torch.bfloat16)
        q_lens = torch.full((shape.batch,), qlen, dtype=torch.int32, device=dev)
        bt = torch.from_numpy(plan.block_table).to(dev)
        lens_d = torch.from_numpy(lens).to(dev)
        max_len = int(lens.max())
        ws = kvq.decode_workspace(kvq.prefill_workspace_size(shape.batch, qlen, shape.num_q_heads, shape.num_kv_heads,
                                                             max_len, shape.page_size), dev)
        out = torch.empty((shape.batch, qlen, shape.num_q_heads, 128), dtype=torch.float32, device=dev)

        def run(i):
            kvq.paged_prefill_attention(q, q_lens, caches[i % 4], bt, lens_d, max_len, shape.hadamard_block,
                                        out=out, workspace=ws, stream=stream)
        for i in range(3):
            run(i)
        ms = _timed(run, 20, stream)
        nbytes = decode_bytes(lens, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
        chunk = kvq.prefill_kernel(shape.batch, qlen, shape.num_q_heads, shape.num_kv_heads) == 1
        rates = _chunk_attention_rates(lens, qlen, shape.num_q_heads, ms)
        if not chunk:  # the split kernel's matrix-core work is not three fp16 passes
            rates = {"attention_TFLOPs": rates["attention_TFLOPs"]}
        rows.append(_line(workload=f"{name} shape, {qlen} queries per sequence "
                                   f"({'speculative verification' if qlen < 16 else 'chunked-prefill chunk'})",
                          batch=shape.batch, queries_per_seq=qlen,
                          kernel="large-chunk (tiles staged per 256 columns)" if chunk else "split (16-column tiles)",
                          attention_ms=round(ms, 5), cache_read_GBps=round(nbytes / ms / 1e6, 1),
                          query_tokens_per_s=round(shape.batch * qlen / (ms * 1e-3), 1), **rates))
        del caches
        torch_empty_cache()
    return rows


def suite_tiny(dev, stream, cpu):
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    shape = W.config("tiny")
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    slots = torch.from_numpy(W.slots_for_positions(plan, shape.page_size, seq, pos)).to(dev)
    k, v = W.draw_kv_device(shape, len(seq), dev)
    cache = kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
    t_pre = _timed(lambda i: kvq.rotate_quantize_append(k, v, slots, cache, shape.hadamard_block, 0, stream=stream),
                   50, stream)
    append, attend, lens = _decode_step_fns(shape, plan, [cache], dev, stream)
    t_step = _timed(lambda i: (append(i), attend(i)), 50, stream)
    # the same calls replayed from a HIP graph (no host launch cost per call)
    t_g_pre = _timed_graph(lambda i: kvq.rotate_quantize_append(k, v, slots, cache, shape.hadamard_block, 0), 20, 10)
    g_append, g_attend, _ = _decode_step_fns(shape, plan, [cache], dev, None)
    t_g_step = _timed_graph(lambda i: (g_append(i), g_attend(i)), 20, 10)
    return [_line(workload="tiny: 1 x 512 tokens, 8/8 heads, Hadamard block 32 (latency)", prefill_append_ms=round(t_pre, 5),
                  decode_step_ms=round(t_step, 5), graph_prefill_append_ms=round(t_g_pre, 5),
                  graph_decode_step_ms=round(t_g_step, 5))]


def _cpu_decode_sample(shape, n_seq):
    """The oracle's decode of the first n_seq sequences (host inputs, a small page plan)."""
    from oracle import kvq_oracle as O
    from paged_decode_attention_amd import workloads as W
    s = shape.with_(batch=n_seq, context_lens=tuple(shape.context_lens[:n_seq]))
    plan = W.plan_pages(s, extra_tokens=0)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.bits)
    O.append(cache, k, v, W.slots_for_positions(plan, s.page_size, seq, pos), s.hadamard_block, s.token_scale)
    q = W.draw_q(s)
    t0 = time.perf_counter()
    O.decode(cache, q, plan.block_table, np.asarray(s.context_lens), s.num_kv_heads, s.hadamard_block)
    dt = time.perf_counter() - t0
    nb = decode_bytes(np.asarray(s.context_lens), s.num_q_heads, s.num_kv_heads, s.bits, s.page_size)
    return {"kind": "oracle", "cores": len(os.sched_getaffinity(0)), "sample": f"decode of {n_seq} sequence(s)",
            "seconds_per_seq": round(dt / n_seq, 3), "GBps": round(nb / dt / 1e9, 4)}


def torch_empty_cache():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_suite(args):
    import torch
    from paged_decode_attention_amd import kvq
    kvq.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    only = {x for x in args.suite_only.split(",") if x}
    for fn in (suite_tiny, suite_sweep, suite_llama2_70b, suite_oscar, suite_pc, suite_multi_query):
        if only and fn.__name__[len("suite_"):] not in only:
            continue
        new = fn(dev, stream, args.suite_cpu)
        for r in new:
            print(json.dumps(r), flush=True)
        rows += new
        torch.cuda.empty_cache()
    return rows


def main():
    args = parse_args()
    if args.summarize_counters:
        cmd = (f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d DIR -o run -- python3 bench.py "
               f"--counters --workload {args.workload} --steps {args.steps} --warmup 0")
        print(summarize_counters(*args.summarize_counters, args.workload, cmd))
        return
    if args.summarize_sq:
        print(summarize_sq(*args.summarize_sq, args.workload))
        return
    if args.summarize_kernel_stats:
        if args.only:  # a trace of one record
            cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- python3 bench.py "
                   f"--only {args.only}")
        elif args.suite_only:  # a trace of suite rows
            cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- python3 bench.py "
                   f"--suite --suite-only {args.suite_only}")
        else:
            cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- python3 bench.py "
                   f"--workload {args.workload} --steps {args.steps} --warmup {args.warmup} --no-cpu-baseline"
                   + (" --no-sub-records" if args.no_sub_records else ""))
        print(summarize_kernel_stats(args.summarize_kernel_stats, cmd))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.suite:
        run_suite(args)
        return
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the kernels run on one GPU's share of the work (one GPU's KV heads "
              "or sequences), and the library has no multi-GPU path; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvq.lib()
    dev = torch.device("cuda:0")
    if args.counters and args.workload in ("llama2_70b", "oscar_int2"):
        counters_other(args, dev)
        return
    if args.only:
        stream = torch.cuda.current_stream()
        if args.only in ("tiny", "sweep"):
            rec = (record_tiny if args.only == "tiny" else record_sweep)(dev, stream)
        else:
            rec = (record_llama2_70b if args.only == "llama2_70b" else record_oscar)(dev, stream, Ceiling(dev))
        print(json.dumps(rec), flush=True)
        return
    shape = W.config(args.workload)
    assert shape.layers == 1 and shape.chunk == 0, "the step benchmark covers single-layer prefill workloads"
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, shape.page_size, seq, pos)
    dseq, dpos = W.decode_positions(shape)
    kn, vn = W.draw_kv(shape, shape.batch, stream="decode")
    dslots = W.slots_for_positions(plan, shape.page_size, dseq, dpos)
    q = W.draw_q(shape)
    lens_dec = np.asarray(shape.context_lens, dtype=np.int32) + 1
    max_len = int(lens_dec.max())

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    k_in = [bf16(k)]
    v_in = [bf16(v)]
    for _ in range(N_INPUT_COPIES - 1):
        k_in.append(k_in[0].clone())
        v_in.append(v_in[0].clone())
    slots_d = torch.from_numpy(slots).to(dev)
    kn_d, vn_d, dslots_d = bf16(kn), bf16(vn), torch.from_numpy(dslots).to(dev)
    q_d = bf16(q)
    bt_d = torch.from_numpy(plan.block_table).to(dev)
    lens_d = torch.from_numpy(lens_dec).to(dev)
    caches = [kvq.PagedKVCache.empty(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.bits, device=dev)
              for _ in range(N_CACHE_COPIES)]
    ws_bytes = kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len,
                                         shape.page_size)
    ws = kvq.decode_workspace(ws_bytes, dev)
    out = torch.empty((shape.batch, shape.num_q_heads, 128), dtype=torch.float32, device=dev)
    hb, ts = shape.hadamard_block, shape.token_scale
    stream = torch.cuda.current_stream()

    def prefill(i):
        kvq.rotate_quantize_append(k_in[i % N_INPUT_COPIES], v_in[i % N_INPUT_COPIES], slots_d,
                                   caches[i % N_CACHE_COPIES], hb, ts, stream=stream)

    def decode_append(i):
        kvq.rotate_quantize_append(kn_d, vn_d, dslots_d, caches[i % N_CACHE_COPIES], hb, ts, stream=stream)

    def attend(c):
        kvq.paged_decode_attention(q_d, caches[c % N_CACHE_COPIES], bt_d, lens_d, max_len, hb, out=out,
                                   workspace=ws, stream=stream)

    def decode_step(c):
        # one launch: append the decode token (position 4096) and attend over 4097 tokens
        kvq.decode_step(q_d, kn_d, vn_d, caches[c % N_CACHE_COPIES], bt_d, lens_d, max_len, hb, token_scale=ts,
                        out=out, workspace=ws, stream=stream)

    # every cache copy holds a full prefill + decode token before anything is timed
    for i in range(N_CACHE_COPIES):
        prefill(i)
        decode_append(i)
    torch.cuda.synchronize()

    def step(i, ev=None):
        # the prefill rewrites copy i; the decode step works on the copy written seven steps ago
        if ev is not None:
            ev[0].record(stream)
        prefill(i)
        if ev is not None:
            ev[1].record(stream)
        decode_step(i + N_CACHE_COPIES // 2)
        if ev is not None:
            ev[2].record(stream)

    if args.counters:
        # calibration copy of known size, then the steps the counters are read on
        src = torch.ones(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        print(f"counters run: 3 calibration copies of {CALIBRATION_BYTES} bytes, {args.steps} steps", flush=True)
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed region: K steps with one event pair around them (no markers between the launches)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps


    # the same K steps again with an event between every launch: per-launch times inside the step (each event
    # adds a marker packet, a few us per launch)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    prefill_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dstep_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    # the prefill append back to back in blocks of 5 launches between events, rotating over the input and
    # cache copies: its launch duration without marker overhead (the roofline's time)
    n_pblk = max(2, args.steps // 5)
    pblk_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_pblk)]
    for j in range(n_pblk):
        pblk_ev[j][0].record(stream)
        for i in range(5):
            prefill(args.warmup + 5 * j + i)
        pblk_ev[j][1].record(stream)
    torch.cuda.synchronize()
    prefill_blk_ms = np.array([e[0].elapsed_time(e[1]) / 5 for e in pblk_ev])

    # the same decode step as two launches (append, then attention), for comparison
    for i in range(5):
        decode_append(i), attend(i)
    torch.cuda.synchronize()
    sep_ms = _timed(lambda i: (decode_append(i), attend(i)), 50, stream)
    fused_ms = _timed(decode_step, 50, stream)

    # decode attention alone, back to back, cycling over the 14 cache copies: blocks of 20
    # launches between events (so event overhead does not enter the per-launch time)
    for i in range(10):
        attend(i)
    torch.cuda.synchronize()
    n_blk = max(1, args.decode_iters // 20)
    blk_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_blk)]
    for j in range(n_blk):
        blk_ev[j][0].record(stream)
        for i in range(20):
            attend(20 * j + i)
        blk_ev[j][1].record(stream)
    torch.cuda.synchronize()
    dec_only_ms = np.array([e[0].elapsed_time(e[1]) / 20 for e in blk_ev])

    b_prefill = append_bytes(len(seq), shape.num_kv_heads, shape.bits)
    b_dapp = append_bytes(shape.batch, shape.num_kv_heads, shape.bits)
    b_attn = decode_bytes(lens_dec, shape.num_q_heads, shape.num_kv_heads, shape.bits, shape.page_size)
    step_bytes = b_prefill + b_dapp + b_attn
    value = step_bytes / (ms_step * 1e-3) / 1e9

    def gbps(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    pre_avg, dstep_avg, dec_avg = float(prefill_blk_ms.mean()), float(dstep_ms.mean()), float(dec_only_ms.mean())
    kernels = {
        "rotate_quantize_append_prefill": {"bytes": b_prefill, "avg_ms": round(pre_avg, 5),
                                           "launches": 5 * n_pblk,
                                           "in_step_event_ms": round(float(prefill_ms.mean()), 5),
                                           "GBps": round(gbps(b_prefill, pre_avg), 1),
                                           "frac_of_peak": round(gbps(b_prefill, pre_avg) / PEAK_HBM_GBPS, 4),
                                           "tokens_per_s": round(len(seq) / (pre_avg * 1e-3), 1),
                                           **_pcts(prefill_blk_ms)},
        "decode_step_fused_in_step": {"bytes": b_dapp + b_attn, "avg_ms": round(dstep_avg, 5),
                                      "GBps": round(gbps(b_dapp + b_attn, dstep_avg), 1),
                                      "note": "kvq_decode_step: decode-token append + attention in one launch"},
        "decode_step_fused_back_to_back": {"bytes": b_dapp + b_attn, "avg_ms": round(fused_ms, 5),
                                           "GBps": round(gbps(b_dapp + b_attn, fused_ms), 1)},
        "decode_step_two_launches": {"bytes": b_dapp + b_attn, "avg_ms": round(sep_ms, 5),
                                     "note": "kvq_rotate_quantize_append of the 16 decode tokens, then "
                                             "kvq_paged_decode_attention"},
        "paged_decode_attention_alone": {
            "bytes": b_attn, "avg_ms": round(dec_avg, 5), "launches": 20 * n_blk,
            "block_median_ms": round(float(np.median(dec_only_ms)), 5),
            "block_p10_ms": round(float(np.percentile(dec_only_ms, 10)), 5),
            "block_p90_ms": round(float(np.percentile(dec_only_ms, 90)), 5),
            "GBps": round(gbps(b_attn, dec_avg), 1), "frac_of_peak": round(gbps(b_attn, dec_avg) / PEAK_HBM_GBPS, 4),
            "decode_tokens_per_s": round(shape.batch / (dec_avg * 1e-3), 1)},
    }
    dominant = "rotate_quantize_append_prefill" if pre_avg >= dec_avg else "paged_decode_attention_alone"
    dom_bytes, dom_ms = (b_prefill, pre_avg) if dominant.startswith("rotate") else (b_attn, dec_avg)
    achieved = gbps(dom_bytes, dom_ms)
    t_app = stored_traffic(shape.name, "append_kernel")
    t_dec = [stored_traffic(shape.name, k) for k in ("decode_mfma_kernel", "decode_merge_splits_kernel")]
    t_dec = None if None in t_dec else sum(t_dec)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": t_app if dominant.startswith("rotate") else t_dec, "kernel": dominant,
                "bytes_per_launch": dom_bytes}
    roofline_decode = {"bound": "hbm", "achieved": round(gbps(b_attn, dec_avg), 1), "peak": PEAK_HBM_GBPS,
                       "unit": "GB/s", "frac": round(gbps(b_attn, dec_avg) / PEAK_HBM_GBPS, 4), "traffic": t_dec,
                       "kernel": "paged_decode_attention (decode + split merge)", "bytes_per_launch": b_attn}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "storage": f"int{shape.bits} codes + fp32 scale/zero",
        "data": "synthetic (seeded bf16 K/V/Q: N(0,1), 4 outlier channels x10, per-token LogNormal(0,1) norms)",
        "config": {"workload": f"{shape.name}: {shape.batch} seq x {shape.context_lens[0]} tokens prefill-append + "
                               f"1 fused decode step (append + attention over {max_len}), {shape.num_q_heads}/"
                               f"{shape.num_kv_heads} heads, head_dim 128, page 16, Hadamard block {hb}, "
                               f"INT{shape.bits}",
                   "global_batch": shape.batch, "seq_len": max_len, "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "step_bytes": step_bytes,
        "decode_tokens_per_s": kernels["paged_decode_attention_alone"]["decode_tokens_per_s"],
        "kernels": kernels, "roofline": roofline, "roofline_decode": roofline_decode,
    }
    # the same decode over an unquantized bf16 cache (the baseline the pages compare against)
    del caches, k_in, v_in
    torch.cuda.empty_cache()
    t_bf, gb_bf = _bf16_attention(shape, plan, dev, stream, n_copies=4)
    result["baseline_bf16_decode"] = {
        "avg_ms": round(t_bf, 5), "GBps": round(gb_bf, 1), "speedup_of_int%d_decode" % shape.bits: round(t_bf / dec_avg, 2),
        "cache_bytes_ratio": round(512 / (2 * 128 * shape.bits // 8 + 16), 2)}
    torch_empty_cache()
    _say(f"{shape.name} step timed")
    if not args.no_sub_records:
        # the practical ceiling at the two kernels' launch shapes
        ceiling = Ceiling(dev)
        c_dec = ceiling.for_decode(b_attn, _decode_waves(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len,
                                                         shape.page_size), stream)
        c_app = ceiling.for_append(len(seq), shape.num_kv_heads, shape.bits, stream,
                                   patterns=("mix", "read", "write", "copy"))
        result["ceiling"] = {"unit": "GB/s", "decode_shape": c_dec, "append_shape": c_app,
                             "note": "streaming probes (libkvq_stream.so) with the kernels' grid, workgroup size and "
                                     "bytes, linear 16-byte accesses; the append's ceiling is its read/write mix"}
        roofline["measured_ceiling"] = c_app["mix"]["GBps"] if dominant.startswith("rotate") else c_dec["GBps"]
        roofline["frac_of_measured_ceiling"] = round(achieved / roofline["measured_ceiling"], 4)
        roofline_decode["measured_ceiling"] = c_dec["GBps"]
        roofline_decode["frac_of_measured_ceiling"] = round(roofline_decode["achieved"] / c_dec["GBps"], 4)
        _say("ceilings measured")
        subs = {}
        subs["tiny"] = record_tiny(dev, stream)
        subs["sweep"] = record_sweep(dev, stream)
        _say("sweep timed")
        subs["llama2_70b"] = record_llama2_70b(dev, stream, ceiling)
        _say("llama2_70b timed")
        subs["oscar_int2"] = record_oscar(dev, stream, ceiling)
        _say("oscar_int2 timed")
        del ceiling
        torch_empty_cache()
        result["sub_records"] = subs
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shape, k, v, slots, plan, q)
        _say(f"{shape.name} CPU oracle timed")
        if not args.no_sub_records:
            subs["tiny"]["cpu_baseline"] = cpu_decode_baseline("tiny", 1)
            for row in subs["sweep"]["rows"]:
                b = row["batch"]
                if b in (1, 8):
                    row["cpu_baseline"] = cpu_decode_baseline(f"sweep_b{b}", b)
                elif b == 32:
                    lens32 = W.config("sweep_b32").context_lens
                    row["cpu_baseline"] = cpu_decode_baseline(
                        "sweep_b32", 8, extrapolate=sum(lens32) / sum(lens32[:8]),
                        note="; scaled to all 32 by their tokens")
            _say("sweep CPU oracle timed")
            subs["llama2_70b"]["cpu_baseline"] = cpu_decode_baseline(
                "llama2_70b", 1, extrapolate=4 * 80, note="; one sequence of one layer, x 4 sequences x 80 layers")
            _say("llama2_70b CPU oracle timed")
            subs["oscar_int2"]["cpu_baseline"] = cpu_decode_baseline(
                "oscar_int2", 4, extrapolate=8, note="; 4 of the 32 sequences, x 8")
            _say("oscar_int2 CPU oracle timed")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

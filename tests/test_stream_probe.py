"""The streaming probe library (libkvq_stream.so, include/kvq_stream.h) that measures the HBM
ceiling: it exports what the header declares and rejects invalid sizes before any launch (host),
and its unit-to-row mapping touches exactly the bytes it is asked to (GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from paged_decode_attention_amd import stream_probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_declared_symbols():
    text = open(os.path.join(ROOT, "include", "kvq_stream.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))
    assert names == sorted(stream_probe.EXPORTS)
    L = stream_probe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_rejects_invalid_sizes():
    L = stream_probe.lib()
    buf = ctypes.create_string_buffer(64)
    p16 = (ctypes.addressof(buf) + 15) // 16 * 16
    sink = ctypes.c_uint32(0)
    sp = ctypes.addressof(sink)

    def call(src=p16, dst=p16, rows=4, rd=1, wr=1, grid=2, block=64, sink=sp, layout=0):
        return L.kvq_stream_probe(src, dst, rows, rd, wr, layout, grid, block, 0, sink, None)
    assert call(rd=0, wr=0) == 1                 # empty rows
    assert call(rows=0) == 1
    assert call(grid=0) == 1
    assert call(block=96) == 1                   # not whole waves
    assert call(block=2048) == 1
    assert call(sink=None) == 1
    assert call(src=None) == 1                   # reads need a source
    assert call(dst=None) == 1                   # writes need a destination
    assert call(src=p16 + 4) == 1                # 16-byte alignment
    assert call(rows=1 << 31, rd=2, wr=0) == 1   # 2^32 units do not fit the 32-bit index
    assert call(layout=2) == 1
    assert call(layout=1, grid=1) == 1           # a reader and a writer workgroup at least


@pytest.mark.gpu
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("rd,wr", [(0, 32), (32, 9), (32, 5), (16, 16)])
def test_every_store_lands_once(rd, wr, layout):
    """Every store position of every row is written exactly once with its position stamp (layout 0:
    (u, r, k, 0) with u = r (rd + wr) + k; layout 1: (r, k, j, 1) with j = r wr + k - rd), and
    nothing past the rows is touched."""
    rows = 3001
    dev = "cuda"
    src = torch.ones(max(rows * rd * 16, 16), dtype=torch.uint8, device=dev)
    dst = torch.full((rows * wr * 16 + 4096,), 0xAB, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"stream probe rows {rows} read {rd} write {wr} layout {layout}", flush=True)
    stream_probe.probe(src, dst, rows, rd, wr, 37 + 41 * layout, 256, sink, layout=layout)
    torch.cuda.synchronize()
    got = dst[:rows * wr * 16].view(torch.int32).cpu().numpy().reshape(rows, wr, 4).astype(np.int64)
    r = np.broadcast_to(np.arange(rows)[:, None], (rows, wr))
    k = np.broadcast_to(rd + np.arange(wr)[None, :], (rows, wr))
    if layout == 0:
        want = np.stack([r * (rd + wr) + k, r, k, np.zeros_like(r)], axis=-1)
    else:
        want = np.stack([r, k, r * wr + k - rd, np.ones_like(r)], axis=-1)
    assert np.array_equal(got, want)
    # nothing past the rows was written
    assert torch.all(dst[rows * wr * 16:] == 0xAB).item()

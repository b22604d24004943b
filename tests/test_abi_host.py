"""The C ABI on the host, without a GPU: the library loads, exports every entry point that
include/kvq.h declares, and rejects invalid arguments with the documented status before any
launch (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

from paged_decode_attention_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = kvq.lib()
    names = _declared()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert kvq.abi_version() == 3


def test_prefill_kernel_choice():
    """The large-chunk kernel is chosen from 128 (query, head) columns per KV head and 256
    workgroups of 128 columns up; other sizes take the split kernel; invalid sizes are rejected."""
    assert kvq.prefill_kernel(32, 512, 28, 4) == 1     # OScaR chunk: 28 x 4 x 32 workgroups
    assert kvq.prefill_kernel(2, 512, 32, 8) == 1      # 16 x 8 x 2 = 256 workgroups
    assert kvq.prefill_kernel(1, 512, 32, 8) == 0      # 128 workgroups: too few to fill the chip
    assert kvq.prefill_kernel(16, 4, 32, 8) == 0       # speculative verification: 16 columns
    assert kvq.prefill_kernel(64, 31, 32, 8) == 0      # 124 columns per KV head
    assert kvq.prefill_kernel(64, 32, 32, 8) == 1      # 128 columns, 512 workgroups
    assert kvq.prefill_kernel(4, 512, 28, 5) == -1     # heads not a multiple
    assert kvq.prefill_kernel(0, 512, 32, 8) == -1


def test_status_strings():
    for s in range(6):
        assert kvq.status_string(s)
    assert kvq.status_string(99) == "unknown status"


NULL = None


def _append(**kw):
    a = dict(k=NULL, v=NULL, ks=1024, vs=1024, n=4, h=8, d=128, slots=NULL, kc=NULL, vc=NULL, ksz=NULL, vsz=NULL,
             pages=10, ps=16, hb=32, bits=4, ts=0)
    a.update(kw)
    return kvq.lib().kvq_rotate_quantize_append(a["k"], a["v"], a["ks"], a["vs"], a["n"], a["h"], a["d"], a["slots"],
                                                a["kc"], a["vc"], a["ksz"], a["vsz"], a["pages"], a["ps"], a["hb"],
                                                a["bits"], a["ts"], NULL)


def test_append_validation():
    assert _append(n=0) == kvq.KVQ_OK                       # no-op before pointer checks
    assert _append() == kvq.KVQ_ERR_NULL
    assert _append(n=-1) == kvq.KVQ_ERR_SHAPE
    assert _append(bits=3) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(bits=8) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(d=64) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(ps=8) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(ps=0) == kvq.KVQ_ERR_SHAPE
    assert _append(hb=3) == kvq.KVQ_ERR_SHAPE
    assert _append(hb=256) == kvq.KVQ_ERR_SHAPE
    assert _append(hb=0) == kvq.KVQ_ERR_SHAPE
    assert _append(ts=2) == kvq.KVQ_ERR_SHAPE
    assert _append(ks=1000) == kvq.KVQ_ERR_SHAPE           # shorter than H * D
    assert _append(ks=1028) == kvq.KVQ_ERR_SHAPE           # not a multiple of 8 elements
    assert _append(h=0) == kvq.KVQ_ERR_SHAPE
    for hb in (1, 2, 4, 8, 16, 32, 64, 128):
        assert _append(hb=hb) == kvq.KVQ_ERR_NULL           # valid sizes: only the pointers are missing


def _decode(**kw):
    a = dict(q=NULL, pre=0, kc=NULL, vc=NULL, ksz=NULL, vsz=NULL, pages=100, ps=16, bt=NULL, mpps=64, cl=NULL,
             mcl=1024, b=2, hq=32, hkv=8, d=128, hb=128, bits=4, scale=0.0, out=NULL, ws=NULL, wsb=0, pps=0)
    a.update(kw)
    return kvq.lib().kvq_paged_decode_attention(
        a["q"], a["pre"], a["kc"], a["vc"], a["ksz"], a["vsz"], a["pages"], a["ps"], a["bt"], a["mpps"], a["cl"],
        a["mcl"], a["b"], a["hq"], a["hkv"], a["d"], a["hb"], a["bits"], a["scale"], a["out"], a["ws"], a["wsb"],
        a["pps"], NULL)


def test_decode_validation():
    assert _decode(b=0) == kvq.KVQ_OK
    assert _decode() == kvq.KVQ_ERR_NULL
    # a context that needs pages with an empty pool is refused before any launch; with no context
    # to read, an empty pool is fine
    assert _decode(pages=0) == kvq.KVQ_ERR_SHAPE
    assert _decode(pages=0, mcl=0) == kvq.KVQ_ERR_NULL
    assert _decode(hq=30) == kvq.KVQ_ERR_SHAPE              # not a multiple of kv heads
    assert _decode(hq=72) == kvq.KVQ_ERR_UNSUPPORTED        # 9 query heads per kv head
    assert _decode(bits=1) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(d=256) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(hb=48) == kvq.KVQ_ERR_SHAPE
    assert _decode(mpps=10) == kvq.KVQ_ERR_SHAPE            # block table narrower than max_context_len needs
    assert _decode(mcl=-1) == kvq.KVQ_ERR_SHAPE
    assert _decode(pre=2) == kvq.KVQ_ERR_SHAPE
    assert _decode(pps=-3) == kvq.KVQ_ERR_SHAPE
    assert _decode(b=-1) == kvq.KVQ_ERR_SHAPE


def test_workspace_size():
    L = kvq.lib()
    # unsplit: no workspace (a batch that fills the waves by itself, sequences of at most 48 pages)
    assert L.kvq_paged_decode_workspace_size(256, 32, 8, 128, 768, 16, 0) == 0
    w = L.kvq_paged_decode_workspace_size(1, 32, 8, 128, 8192, 16, 0)
    assert w > 0
    # forced split size: splits = ceil(512 / 64) = 8 -> 8 * 32 * 130 floats at least
    w8 = L.kvq_paged_decode_workspace_size(1, 32, 8, 128, 8192, 16, 64)
    assert w8 >= 8 * 32 * 130 * 4
    assert L.kvq_paged_decode_workspace_size(1, 32, 8, 128, 8192, 16, 512) == 0   # one split
    assert L.kvq_paged_decode_workspace_size(0, 32, 8, 128, 8192, 16, 0) == 0
    # the bf16 baseline's split partials: 8 splits x 32 rows of 128 floats and (max, sum) pairs
    assert L.kvq_paged_decode_bf16_workspace_size(1, 32, 8, 128, 8192, 16, 64) == 8 * 32 * 128 * 4 + 8 * 32 * 8
    assert L.kvq_paged_decode_bf16_workspace_size(1, 32, 8, 128, 8192, 16, 512) == 0


def _splits(batch, hq, hkv, max_len, pps=0):
    """Number of splits the library plans, read back from the workspace size (acc + (m, l) rows)."""
    w = kvq.lib().kvq_paged_decode_workspace_size(batch, hq, hkv, 128, max_len, 16, pps)
    per_split = batch * hq * 128 * 4
    return round(w / (per_split + batch * hq * 8)) if w else 1


def test_split_plan():
    # Llama-3-8B decode, 4097 tokens (257 pages), 16 x 8 (sequence, KV head) items: 16 even splits of
    # 16 pages, the 257th page joining the last split
    assert _splits(16, 32, 8, 4097) == 16
    assert _splits(16, 32, 8, 4096) == 16
    # a remainder of more than half a split gets its own split: 16 * 16 + 9 pages
    assert _splits(16, 32, 8, (16 * 16 + 9) * 16) == 17
    # Llama-2-70B, 32769 tokens (2049 pages), 4 x 8 items: 64 splits of 32 pages
    assert _splits(4, 64, 8, 32769) == 64
    # enough (sequence, KV head) items to fill the GPU: no split while a sequence fits in 48 pages,
    # else splits of at most 48 pages (513 pages: 10 of 48, the remaining 33 more than half of one)
    assert _splits(256, 32, 8, 768) == 1
    assert _splits(256, 32, 8, 8193) == 11
    # 32 sequences x 8 heads: the 8 splits of 64 pages that fill the waves become 48-page splits
    assert _splits(32, 32, 8, 8193) == 11
    # 16 x 8 items with 1025 pages: 16 splits of 64 pages (more than 8 per sequence: no cap)
    assert _splits(16, 28, 4, 16385) == 32 and _splits(32, 28, 4, 16385) == 16
    # a forced split size is taken literally
    assert _splits(1, 32, 8, 4097, pps=16) == 17
    assert _splits(1, 32, 8, 4097, pps=1) == 257


def test_dequant_validation():
    L = kvq.lib()
    f = lambda **kw: L.kvq_dequant_page(NULL, NULL, kw.get("t", 0), kw.get("page", 0), kw.get("pages", 4), 8, 16, 128,
                                        kw.get("hb", 32), kw.get("bits", 4), kw.get("un", 0), NULL, NULL)
    assert f() == kvq.KVQ_ERR_NULL
    assert f(page=4) == kvq.KVQ_ERR_SHAPE
    assert f(page=-1) == kvq.KVQ_ERR_SHAPE
    assert f(t=2) == kvq.KVQ_ERR_SHAPE
    assert f(un=5) == kvq.KVQ_ERR_SHAPE
    assert f(bits=3) == kvq.KVQ_ERR_UNSUPPORTED


def test_binding_refuses_host_tensors():
    import torch
    c = kvq.PagedKVCache.empty(4, 2, 16, 4, device="cpu")
    with pytest.raises(ValueError):
        kvq.dequant_page(c, "k", 0, 32)
    # a caller's workspace must be device memory too (its pointer goes to the kernels)
    with pytest.raises(ValueError):
        kvq._workspace(torch.empty(64, dtype=torch.uint8))
    assert kvq._workspace(None) == (None, 0)


def test_bf16_baseline_validation():
    L = kvq.lib()
    w = lambda **kw: L.kvq_bf16_cache_write(NULL, NULL, kw.get("ks", 1024), 1024, kw.get("n", 4), 8, kw.get("d", 128),
                                            NULL, NULL, NULL, 10, kw.get("ps", 16), NULL)
    assert w() == kvq.KVQ_ERR_NULL
    assert w(n=0) == kvq.KVQ_OK
    assert w(d=64) == kvq.KVQ_ERR_UNSUPPORTED
    assert w(ps=24) == kvq.KVQ_ERR_UNSUPPORTED
    assert w(ks=1000) == kvq.KVQ_ERR_SHAPE

    def dec(**kw):
        return L.kvq_paged_decode_attention_bf16(
            NULL, NULL, NULL, kw.get("pages", 10), 16, NULL, kw.get("mp", 4), NULL, kw.get("ml", 64), kw.get("b", 2),
            kw.get("hq", 32), kw.get("hkv", 8), 128, 0.0, NULL, NULL, 0, 0, NULL)
    assert dec() == kvq.KVQ_ERR_NULL
    assert dec(pages=0) == kvq.KVQ_ERR_SHAPE          # pages to read, an empty pool
    assert dec(pages=0, ml=0) == kvq.KVQ_ERR_NULL
    assert dec(b=0) == kvq.KVQ_OK
    assert dec(hq=30) == kvq.KVQ_ERR_SHAPE            # not a multiple of the KV heads
    assert dec(hq=136) == kvq.KVQ_ERR_UNSUPPORTED     # 17 query heads per KV head
    assert dec(mp=3) == kvq.KVQ_ERR_SHAPE             # block table too narrow for 64 tokens


def test_decode_step_validation():
    L = kvq.lib()

    def step(**kw):
        return L.kvq_decode_step(
            NULL, 0, NULL, NULL, kw.get("ks", 1024), 1024, NULL, NULL, NULL, NULL, 10, 16, NULL, 4, NULL, 64,
            kw.get("b", 2), 32, 8, 128, kw.get("hb", 128), kw.get("bits", 4), kw.get("ts", 0), 0.0, NULL, NULL, 0, 0,
            NULL)
    assert step() == kvq.KVQ_ERR_NULL
    assert step(b=0) == kvq.KVQ_OK
    assert step(bits=3) == kvq.KVQ_ERR_UNSUPPORTED
    assert step(ts=2) == kvq.KVQ_ERR_SHAPE
    assert step(ks=1000) == kvq.KVQ_ERR_SHAPE


def test_prefill_validation_and_workspace():
    L = kvq.lib()

    def pre(**kw):
        return L.kvq_paged_prefill_attention(
            NULL, 0, NULL, kw.get("ql", 4), NULL, NULL, NULL, NULL, 10, 16, NULL, 4, NULL, 64, kw.get("b", 2),
            kw.get("hq", 32), 8, 128, 128, kw.get("bits", 4), 0.0, NULL, NULL, 0, 0, NULL)
    assert pre() == kvq.KVQ_ERR_NULL
    assert pre(b=0) == kvq.KVQ_OK
    assert pre(ql=0) == kvq.KVQ_ERR_SHAPE
    assert pre(hq=30) == kvq.KVQ_ERR_SHAPE
    assert pre(bits=3) == kvq.KVQ_ERR_UNSUPPORTED
    assert pre(hq=8 * 24) == kvq.KVQ_ERR_NULL      # 24 heads per KV head are fine with several queries
    # workspace: one split when the (sequence, KV head, column tile) items fill the GPU
    assert L.kvq_paged_prefill_workspace_size(64, 16, 32, 8, 128, 4096, 16, 0) == 0
    w = L.kvq_paged_prefill_workspace_size(1, 4, 32, 8, 128, 4096, 16, 0)
    assert w >= 2 * 4 * 32 * 130 * 4


def _pc_write(**kw):
    a = dict(k=NULL, v=NULL, ks=1024, vs=1024, n=2, ids=NULL, h=8, d=128, kc=NULL, vc=NULL, kss=NULL, vss=NULL,
             kcp=NULL, vcp=NULL, pages=10, ps=32, hb=128, bits=2)
    a.update(kw)
    return kvq.lib().kvq_pc_write_pages(a["k"], a["v"], a["ks"], a["vs"], a["n"], a["ids"], a["h"], a["d"], a["kc"],
                                        a["vc"], a["kss"], a["vss"], a["kcp"], a["vcp"], a["pages"], a["ps"], a["hb"],
                                        a["bits"], NULL)


def _pc_decode(**kw):
    a = dict(q=NULL, kc=NULL, vc=NULL, kss=NULL, vss=NULL, kcp=NULL, vcp=NULL, pages=10, ps=64, bt=NULL, mp=8,
             cl=NULL, mcl=500, tk=NULL, tv=NULL, b=2, hq=32, hkv=8, d=128, hb=128, bits=4, ss=0.0, out=NULL,
             ws=NULL, wsb=0, pps=0)
    a.update(kw)
    return kvq.lib().kvq_pc_decode_attention(
        a["q"], a["kc"], a["vc"], a["kss"], a["vss"], a["kcp"], a["vcp"], a["pages"], a["ps"], a["bt"], a["mp"],
        a["cl"], a["mcl"], a["tk"], a["tv"], a["b"], a["hq"], a["hkv"], a["d"], a["hb"], a["bits"], a["ss"], a["out"],
        a["ws"], a["wsb"], a["pps"], NULL)


def test_pc_validation_and_workspace():
    assert _pc_decode(pages=0) == kvq.KVQ_ERR_SHAPE       # complete pages to read, an empty pool
    assert _pc_decode(pages=0, mcl=63) == kvq.KVQ_ERR_NULL  # only the unfinished page (the tail)
    assert _pc_write(n=0) == kvq.KVQ_OK
    assert _pc_write() == kvq.KVQ_ERR_NULL
    assert _pc_write(n=-1) == kvq.KVQ_ERR_SHAPE
    assert _pc_write(ps=16) == kvq.KVQ_ERR_UNSUPPORTED      # per-channel pages are 32, 64 or 128 tokens
    assert _pc_write(ps=256) == kvq.KVQ_ERR_UNSUPPORTED
    assert _pc_write(ps=48) == kvq.KVQ_ERR_UNSUPPORTED
    assert _pc_write(bits=3) == kvq.KVQ_ERR_UNSUPPORTED
    assert _pc_write(hb=3) == kvq.KVQ_ERR_SHAPE
    assert _pc_write(ks=1000) == kvq.KVQ_ERR_SHAPE          # stride below one token's heads
    assert _pc_write(ks=1028) == kvq.KVQ_ERR_SHAPE          # stride not a multiple of 8
    # one grid dimension of 4 page_size threads per (page, head): 2^22 pages x 8 heads x 32 = 2^30
    assert _pc_write(n=1 << 22) == kvq.KVQ_ERR_UNSUPPORTED
    assert _pc_write(n=(1 << 22) - 1) == kvq.KVQ_ERR_NULL
    assert _pc_decode(b=0) == kvq.KVQ_OK
    assert _pc_decode() == kvq.KVQ_ERR_NULL
    assert _pc_decode(ps=16) == kvq.KVQ_ERR_UNSUPPORTED
    assert _pc_decode(hq=31) == kvq.KVQ_ERR_SHAPE
    assert _pc_decode(hq=72) == kvq.KVQ_ERR_UNSUPPORTED     # 9 query heads per KV head
    assert _pc_decode(mp=6) == kvq.KVQ_ERR_SHAPE            # 500 // 64 = 7 complete pages need 7 entries
    assert _pc_decode(mp=7, b=0) == kvq.KVQ_OK
    # workspace: page splits over the complete pages plus the tail split, (splits + 1) rows each
    ws = kvq.lib().kvq_pc_decode_workspace_size
    one = ws(1, 4, 1, 128, 63, 64, 0)                       # no complete page: one empty page split + the tail
    assert one == 2 * 4 * 128 * 4 + 256                     # two splits of 4 rows (acc), then (max, sum) rounded up
    assert ws(2, 32, 8, 128, 4096, 64, 0) > ws(2, 32, 8, 128, 4096, 64, 64)
    assert ws(2, 32, 8, 128, 4096, 64, 64) == 2 * 2 * 32 * 128 * 4 + 1024   # 128 rows of (max, sum)
    assert ws(0, 32, 8, 128, 4096, 64, 0) == 0


def test_launch_grid_limits():
    # a launch dimension holds fewer than 2^32 work-items: larger sizes are refused before any
    # pointer is looked at (NULL pointers below), sizes just inside pass on to the pointer checks
    # append: one 64-lane wave per (16-token tile, KV head) item, four items per 256-thread workgroup
    assert _append(n=16 * (1 << 24), h=4, ks=512, vs=512) == kvq.KVQ_ERR_UNSUPPORTED            # 2^26 items
    assert _append(n=16 * ((1 << 24) - 1), h=4, ks=512, vs=512) == kvq.KVQ_ERR_NULL             # 2^26 - 4
    # decode: one wave per (split, sequence, KV head) (here one page per split) and one merge wave
    # per (sequence, head)
    big = 16 * (1 << 26)  # 2^26 pages of 16 tokens
    one = dict(b=1, hq=4, hkv=1, mpps=1 << 26, pps=1, pages=1 << 26)
    assert _decode(mcl=big - 16, **one) == kvq.KVQ_ERR_NULL                                       # 2^26 - 1 splits
    assert _decode(mcl=big, **one) == kvq.KVQ_ERR_UNSUPPORTED                                     # 2^26 splits
    assert _decode(mcl=16 * (1 << 22), mpps=1 << 22, pps=1, pages=1 << 22) == kvq.KVQ_ERR_UNSUPPORTED  # 2^22 x 16 items
    assert _decode(b=65535, hq=1025, hkv=205, mcl=64, mpps=4) == kvq.KVQ_ERR_UNSUPPORTED          # > 2^26 pairs
    assert _decode(b=65535, hq=1020, hkv=204, mcl=64, mpps=4) == kvq.KVQ_ERR_NULL                 # < 2^26 pairs

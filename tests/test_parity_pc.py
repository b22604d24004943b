"""GPU parity of the per-channel pages (kvq_pc_write_pages, kvq_pc_decode_attention) against the
CPU oracle (``write_pages_pc``, ``decode_pc``).

The write test compares a GPU-written cache with the oracle's element by element (codes exact
except next to a rounding boundary, token scales and channel (scale, zero) to float32
accuracy, untouched pages still poison). The decode tests run the GPU read path on the oracle's
own cache, uploaded, so both sides see the same bytes; one test chains the GPU write into the
GPU decode. Each case prints its name and shape before touching the GPU.
"""
import numpy as np
import pytest
import torch

import parity_helpers as H
from oracle import kvq_oracle as O
from paged_decode_attention_amd import kvq
from paged_decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _case(shape, ps, bits, hb, seed, spare_pages=3):
    """Sequences of shape.context_lens tokens: their complete pages written by the oracle into
    shuffled pages of a per-channel cache, their tails, and the block table."""
    lens = list(shape.context_lens)
    n_full = [n // ps for n in lens]
    total = sum(lens)
    k, v = W.draw_kv(shape, max(total, 1))
    rng = np.random.default_rng(seed)
    num_pages = sum(n_full) + spare_pages
    order = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((len(lens), max(1, max(n_full))), -1, dtype=np.int32)
    tail_k = np.zeros((len(lens), ps, shape.num_kv_heads, 128), dtype=np.uint16)
    tail_v = np.zeros_like(tail_k)
    pk, pv, ids = [], [], []
    start, nxt = 0, 0
    for b, n in enumerate(lens):
        for j in range(n // ps):
            bt[b, j] = order[nxt]
            ids.append(order[nxt])
            nxt += 1
            pk.append(k[start + j * ps:start + (j + 1) * ps])
            pv.append(v[start + j * ps:start + (j + 1) * ps])
        full = (n // ps) * ps
        tail_k[b, :n - full] = k[start + full:start + n]
        tail_v[b, :n - full] = v[start + full:start + n]
        start += n
    pk = np.concatenate(pk) if pk else np.zeros((0, shape.num_kv_heads, 128), np.uint16)
    pv = np.concatenate(pv) if pv else np.zeros((0, shape.num_kv_heads, 128), np.uint16)
    ids = np.array(ids, dtype=np.int32)
    cache = O.PagedCachePC(num_pages, shape.num_kv_heads, ps, 128, bits)
    diag = O.write_pages_pc(cache, pk, pv, ids, hb) if len(ids) else None
    return dict(cache=cache, bt=bt, tail_k=tail_k, tail_v=tail_v, pk=pk, pv=pv, ids=ids, diag=diag, lens=lens)


def _upload(c: O.PagedCachePC) -> kvq.PagedKVCachePC:
    d = H.to_dev
    return kvq.PagedKVCachePC(d(c.k_codes), d(c.v_codes), d(c.k_s), d(c.v_s), d(c.k_cp), d(c.v_cp), c.bits)


def _poisoned(num_pages, kv_heads, ps, bits) -> kvq.PagedKVCachePC:
    c = kvq.PagedKVCachePC.empty(num_pages, kv_heads, ps, bits)
    for t in (c.k_codes, c.v_codes):
        t.fill_(0xAA)
    for t in (c.k_s, c.v_s, c.k_cp, c.v_cp):
        t.fill_(float("nan"))
    return c


def _download(dev: kvq.PagedKVCachePC) -> O.PagedCachePC:
    p, h, ps, _ = dev.k_codes.shape
    c = O.PagedCachePC(p, h, ps, 128, dev.bits, poison=False)
    for name in ("k_codes", "v_codes", "k_s", "v_s", "k_cp", "v_cp"):
        getattr(c, name)[:] = getattr(dev, name).cpu().numpy()
    return c


def _compare_pc_caches(got: O.PagedCachePC, ref: O.PagedCachePC, ids, diag, what):
    bits = ref.bits
    written = np.zeros(ref.num_pages, dtype=bool)
    written[ids] = True
    assert np.all(got.k_codes[~written] == 0xAA) and np.all(got.v_codes[~written] == 0xAA), f"{what}: stray code writes"
    for name in ("k_s", "v_s", "k_cp", "v_cp"):
        assert np.all(np.isnan(getattr(got, name)[~written])), f"{what}: stray {name} writes"
    n_bad = 0
    for i, page in enumerate(ids):
        for h in range(ref.kv_heads):
            for tensor in ("k", "v"):
                gc, gs, gcp = got.read_page(page, h, tensor)
                rc, rs, rcp = ref.read_page(page, h, tensor)
                n_bad += H.check_codes(gc, rc, diag[f"{tensor}_t"][i, h], f"{what} {tensor} page {page} head {h}")
                assert np.all(np.abs(gs.astype(np.float64) - rs) <= 1e-6 * np.abs(rs)), f"{what}: {tensor} token scales"
                H.check_scale_zero(gcp[0], gcp[1], rcp[0], rcp[1], bits, f"{what} {tensor} page {page} head {h}")
    _say(f"  {what}: {len(ids)} pages, boundary mismatches {n_bad}")


@pytest.mark.parametrize("ps", [32, 64, 128])
@pytest.mark.parametrize("bits,hb", [(2, 128), (4, 128), (4, 32), (2, 1)])
def test_pc_write(ps, bits, hb):
    shape = W.config("oscar_int2", batch=3, num_q_heads=28, num_kv_heads=4).with_(context_lens=(2 * ps + 5, ps, 3 * ps))
    _say(f"pc write: page {ps}, INT{bits}, Hadamard block {hb}, lens {shape.context_lens}")
    c = _case(shape, ps, bits, hb, seed=ps + bits + hb)
    dev = _poisoned(c["cache"].num_pages, shape.num_kv_heads, ps, bits)
    kvq.pc_write_pages(H.to_dev_bf16(c["pk"]), H.to_dev_bf16(c["pv"]), H.to_dev(c["ids"]), dev, hb)
    torch.cuda.synchronize()
    _compare_pc_caches(_download(dev), c["cache"], c["ids"], c["diag"], f"ps{ps} INT{bits} b{hb}")


def test_pc_write_skips_out_of_range_pages_and_strided_input():
    ps, bits, hb = 32, 4, 128
    shape = W.config("llama3_8b", batch=1, num_q_heads=8, num_kv_heads=2).with_(context_lens=(3 * ps,))
    _say("pc write: ids -1 and num_pages skipped, token stride wider than the heads")
    c = _case(shape, ps, bits, hb, seed=5)
    ids = c["ids"].copy()
    ids[1] = -1
    ref = O.PagedCachePC(c["cache"].num_pages, 2, ps, 128, bits)
    diag = O.write_pages_pc(ref, c["pk"], c["pv"], ids, hb)
    ids_dev = ids.copy()
    ids_dev[1] = c["cache"].num_pages   # out of range on the device side, skipped like -1
    big_k = torch.zeros((3 * ps, 5, 128), dtype=torch.bfloat16, device="cuda")
    big_k[:, :2] = H.to_dev_bf16(c["pk"])
    dev = _poisoned(c["cache"].num_pages, 2, ps, bits)
    kvq.pc_write_pages(big_k[:, :2], H.to_dev_bf16(c["pv"]), H.to_dev(ids_dev), dev, hb)
    torch.cuda.synchronize()
    keep = ids >= 0
    _compare_pc_caches(_download(dev), ref, ids[keep], {t: diag[t][keep] for t in diag}, "skip/stride")


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that bf16 holds exactly -> bf16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _degenerate_pages(ps, heads, seed):
    """Five input pages of small integers times a power of two: (0) every token the same vector,
    so every channel is constant; (1) two all-zero tokens; (2) magnitudes near 2^-120, so the token
    RMS is below 2^-100; (3) magnitudes near 2^100, RMS above 2^100; (4) every token a permutation of
    one multiset of values, channels 0-15 set to one value, so all tokens share one RMS and (for
    block size 1) sixteen channels are constant."""
    rng = np.random.default_rng(seed)
    pages = []
    ints = lambda *shape: rng.integers(-8, 9, size=shape).astype(np.float32)  # noqa: E731
    base = ints(1, heads, 128)
    pages.append(np.repeat(base, ps, axis=0))
    p1 = ints(ps, heads, 128)
    p1[3] = 0.0
    p1[ps - 1] = 0.0
    pages.append(p1)
    pages.append(ints(ps, heads, 128) * np.float32(2.0 ** -120))
    pages.append(ints(ps, heads, 128) * np.float32(2.0 ** 100))
    vals = ints(heads, 128)
    vals[:, :16] = 3.0
    p4 = np.empty((ps, heads, 128), np.float32)
    for t in range(ps):
        for h in range(heads):
            p4[t, h, :16] = 3.0
            p4[t, h, 16:] = rng.permutation(vals[h, 16:])
    pages.append(p4)
    return _bf16_bits(np.concatenate(pages))


@pytest.mark.parametrize("bits,hb", [(4, 1), (2, 1), (4, 128), (2, 32)])
def test_pc_write_degenerate_pages(bits, hb):
    ps, heads = 32, 2
    _say(f"pc write degenerate pages: page {ps}, INT{bits}, Hadamard block {hb}")
    pk = _degenerate_pages(ps, heads, seed=11)
    pv = _degenerate_pages(ps, heads, seed=12)
    ids = np.array([4, 0, 6, 2, 5], dtype=np.int32)
    ref = O.PagedCachePC(7, heads, ps, 128, bits)
    diag = O.write_pages_pc(ref, pk, pv, ids, hb)
    dev = _poisoned(7, heads, ps, bits)
    kvq.pc_write_pages(H.to_dev_bf16(pk), H.to_dev_bf16(pv), H.to_dev(ids), dev, hb)
    torch.cuda.synchronize()
    got = _download(dev)
    _compare_pc_caches(got, ref, ids, diag, f"degenerate INT{bits} b{hb}")
    # the constant page: zero codes, zero scales, the channel value as zero point
    for tensor in ("k", "v"):
        gc, _, gcp = got.read_page(int(ids[0]), 0, tensor)
        assert np.all(gc == 0) and np.all(gcp[0] == 0), f"{tensor}: constant page gives nonzero codes or scales"


def _decode_case(name, shape, ps, bits, hb, pps_list, seed, heads=None):
    c = _case(shape, ps, bits, hb, seed=seed)
    q = W.draw_q(shape)
    lens = np.array(c["lens"], dtype=np.int32)
    max_len = int(lens.max()) if len(lens) else 0
    ref = O.decode_pc(c["cache"], q, c["bt"], lens, c["tail_k"], c["tail_v"], shape.num_kv_heads, hb, heads=heads)
    dev = _upload(c["cache"])
    for pps in pps_list:
        _say(f"pc decode {name}: page {ps}, INT{bits}, b {hb}, pages_per_split {pps}")
        got = kvq.pc_decode_attention(H.to_dev_bf16(q), dev, H.to_dev(c["bt"]), H.to_dev(lens), max_len,
                                      H.to_dev_bf16(c["tail_k"]), H.to_dev_bf16(c["tail_v"]), hb,
                                      pages_per_split=pps)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        if heads is None:
            H.check_attention(got, ref, f"{name} pps {pps}")
            for b, n in enumerate(c["lens"]):
                if n == 0:
                    assert np.all(got[b] == 0), f"{name}: empty sequence gives nonzero output"
        else:
            H.check_attention(got, ref, f"{name} pps {pps}", heads=heads)


@pytest.mark.parametrize("ps", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 4])
def test_pc_decode_ragged(ps, bits):
    # empty, tail only, exact pages, pages + tail, one token; g = 7 (28 / 4 heads)
    lens = (0, ps - 1, 4 * ps, 5 * ps + 17, 1, 2 * ps + ps // 2)
    shape = W.config("oscar_int2", batch=len(lens), num_q_heads=28, num_kv_heads=4).with_(context_lens=lens)
    _decode_case("ragged", shape, ps, bits, 128, [0, 1, 3, 1000], seed=ps * bits)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8)])
def test_pc_decode_group_sizes(hq, hkv):
    ps = 64
    lens = (700, 64, 129)
    shape = W.config("llama3_8b", batch=3, num_q_heads=hq, num_kv_heads=hkv).with_(context_lens=lens)
    _decode_case(f"g{hq // hkv}", shape, ps, 4, 128, [0, 2], seed=hq)


def test_pc_decode_plain_int_and_small_block():
    lens = (300, 77)
    for hb in (1, 16):
        shape = W.config("llama3_8b", batch=2, num_q_heads=16, num_kv_heads=4).with_(context_lens=lens)
        _decode_case(f"b{hb}", shape, 32, 4, hb, [0], seed=hb)


def test_pc_write_then_decode_on_gpu():
    """The GPU-written cache read by the GPU decode matches the oracle's decode of the oracle's cache
    (the two caches differ only in boundary codes, within the attention tolerance)."""
    ps, bits, hb = 64, 2, 128
    lens = (1000, 333, 64)
    shape = W.config("oscar_int2", batch=3, num_q_heads=28, num_kv_heads=4).with_(context_lens=lens)
    _say("pc write then decode, both on the GPU")
    c = _case(shape, ps, bits, hb, seed=77)
    dev = _poisoned(c["cache"].num_pages, shape.num_kv_heads, ps, bits)
    kvq.pc_write_pages(H.to_dev_bf16(c["pk"]), H.to_dev_bf16(c["pv"]), H.to_dev(c["ids"]), dev, hb)
    q = W.draw_q(shape)
    lens_a = np.array(lens, dtype=np.int32)
    got = kvq.pc_decode_attention(H.to_dev_bf16(q), dev, H.to_dev(c["bt"]), H.to_dev(lens_a), int(lens_a.max()),
                                  H.to_dev_bf16(c["tail_k"]), H.to_dev_bf16(c["tail_v"]), hb)
    torch.cuda.synchronize()
    ref = O.decode_pc(c["cache"], q, c["bt"], lens_a, c["tail_k"], c["tail_v"], shape.num_kv_heads, hb)
    H.check_attention(got.cpu().numpy(), ref, "write+decode")


def test_pc_decode_sampled_large():
    """A Llama-3-8B-sized layer (16 sequences of 4097 tokens, 32/8 heads) on per-channel INT2 pages
    of 64 tokens, in the library's own split choice; sampled heads against the oracle."""
    ps = 64
    shape = W.config("llama3_8b").with_(context_lens=(4097,) * 16)
    rng = np.random.default_rng(9)
    heads = [(int(b), int(h)) for b, h in zip(rng.integers(0, 16, 12), rng.integers(0, 32, 12))]
    _decode_case("llama3_8b-sized", shape, ps, 2, 128, [0], seed=11, heads=heads)


def _pc_random_config(i):
    r = np.random.default_rng(8000 + i)
    ps = int(r.choice([32, 64, 128]))
    bits = int(r.choice([2, 4]))
    hb = int(2 ** int(r.integers(0, 8)))
    kvh = int(r.choice([1, 2, 4]))
    g = int(r.integers(1, 9))
    b = int(r.integers(1, 4))
    lens = [int(n) if r.random() > 0.15 else 0 for n in r.integers(1, 4 * ps, size=b)]
    if max(lens) == 0:
        lens[0] = int(r.integers(1, 4 * ps))
    pps = int(r.choice([0, 1, 2, 1000]))
    shape = W.config("oscar_int2", batch=b, num_q_heads=kvh * g, num_kv_heads=kvh,
                     seed=8000 + i).with_(context_lens=tuple(lens))
    return shape, ps, bits, hb, pps


@pytest.mark.parametrize("i", range(12))
def test_pc_random_configuration(i):
    """Seeded random shapes (page size, width, block size, heads, group size, ragged lengths with
    tails and empty sequences, split size): the GPU page writer against the oracle's pages, then the
    GPU decode over the oracle's pages and tails against the oracle's decode."""
    shape, ps, bits, hb, pps = _pc_random_config(i)
    _say(f"pc random {i}: lens {shape.context_lens}, heads {shape.num_q_heads}/{shape.num_kv_heads}, page {ps}, "
         f"INT{bits}, block {hb}, pages_per_split {pps}")
    c = _case(shape, ps, bits, hb, seed=8000 + i)
    if len(c["ids"]):
        dev = _poisoned(c["cache"].num_pages, shape.num_kv_heads, ps, bits)
        kvq.pc_write_pages(H.to_dev_bf16(c["pk"]), H.to_dev_bf16(c["pv"]), H.to_dev(c["ids"]), dev, hb)
        torch.cuda.synchronize()
        _compare_pc_caches(_download(dev), c["cache"], c["ids"], c["diag"], f"random {i}")
    _decode_case(f"random {i}", shape, ps, bits, hb, [pps], seed=8000 + i)

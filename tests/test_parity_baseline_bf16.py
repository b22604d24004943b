"""GPU parity of the bf16 baseline (kvq_bf16_cache_write, kvq_paged_decode_attention_bf16)
against the CPU oracle's bf16 paged cache and decode."""
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


def _poisoned(num_pages, kv_heads, page_size):
    c = kvq.PagedKVCacheBF16.empty(num_pages, kv_heads, page_size)
    c.k.view(torch.int16).fill_(0x7FC0)   # bf16 NaN
    c.v.view(torch.int16).fill_(0x7FC0)
    return c


def _upload(host: O.PagedCacheBF16) -> kvq.PagedKVCacheBF16:
    return kvq.PagedKVCacheBF16(H.to_dev(host.k.view(np.int16)).view(torch.bfloat16),
                                H.to_dev(host.v.view(np.int16)).view(torch.bfloat16))


def _oracle_cache(shape, lens, plan=None):
    s = shape.with_(context_lens=tuple(lens))
    plan = plan or W.plan_pages(s, extra_tokens=0)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCacheBF16(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim)
    O.append_bf16(cache, k, v, W.slots_for_positions(plan, s.page_size, seq, pos))
    return s, plan, cache


def _gpu_decode(shape, plan, dev_cache, q, lens, pps=0):
    max_len = int(max(lens)) if len(lens) else 0
    nbytes = kvq.decode_bf16_workspace_size(len(lens), shape.num_q_heads, shape.num_kv_heads, max_len,
                                            shape.page_size, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")   # contents must not matter
    out = kvq.paged_decode_attention_bf16(H.to_dev_bf16(q), dev_cache, H.to_dev(plan.block_table),
                                          H.to_dev(np.asarray(lens, dtype=np.int32)), max_len, workspace=ws,
                                          pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("page_size", [16, 32])
def test_bf16_cache_write_bit_exact(page_size):
    shape = W.config("tiny", batch=3, num_q_heads=8, num_kv_heads=4, context_lens=(40, 7, 33), page_size=page_size)
    _say(f"bf16 cache write, page size {page_size}")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, page_size, seq, pos)
    slots[5] = -1                                   # skipped
    slots[9] = plan.num_pages * page_size + 3       # outside the pool: skipped
    ref = O.PagedCacheBF16(plan.num_pages, 4, page_size, 128)
    O.append_bf16(ref, k, v, slots)
    dev = _poisoned(plan.num_pages, 4, page_size)
    kvq.bf16_cache_write(H.to_dev_bf16(k), H.to_dev_bf16(v), H.to_dev(slots), dev)
    torch.cuda.synchronize()
    assert np.array_equal(dev.k.view(torch.int16).cpu().numpy().view(np.uint16), ref.k)
    assert np.array_equal(dev.v.view(torch.int16).cpu().numpy().view(np.uint16), ref.v)


CASES = [
    ("tiny", {}, (512,)),
    ("llama3_8b", dict(batch=4), (0, 1, 37, 300)),
    ("llama2_70b", dict(batch=2), (700, 129)),
    ("oscar_int2", dict(batch=3), (500, 16, 250)),
    ("sweep_b8", dict(batch=3), (17, 256, 511)),
]


@pytest.mark.parametrize("name,overrides,lens", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("pps", [0, 1, 3, 1000])
def test_bf16_decode_parity(name, overrides, lens, pps):
    shape = W.config(name, **overrides)
    _say(f"bf16 decode {name} lens={lens} pages_per_split={pps}")
    s, plan, cache = _oracle_cache(shape, lens)
    q = W.draw_q(s)
    ref = O.decode_bf16(cache, q, plan.block_table, np.array(lens), s.num_kv_heads)
    got = _gpu_decode(s, plan, _upload(cache), q, lens, pps=pps)
    worst = H.check_attention(got, ref, f"bf16 {name}/pps{pps}")
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)
    _say(f"  worst rel-L2 {worst:.2e}")


@pytest.mark.parametrize("g", [1, 3, 8, 16])
def test_bf16_decode_group_sizes(g):
    shape = W.config("llama3_8b", batch=2, num_q_heads=2 * g, num_kv_heads=2)
    lens = (150, 33)
    _say(f"bf16 decode GQA group {g}")
    s, plan, cache = _oracle_cache(shape, lens)
    q = W.draw_q(s)
    ref = O.decode_bf16(cache, q, plan.block_table, np.array(lens), 2)
    H.check_attention(_gpu_decode(s, plan, _upload(cache), q, lens, pps=2), ref, f"bf16 g{g}")


def test_bf16_decode_full_llama3_8b_sampled():
    shape = W.config("llama3_8b")
    lens = shape.context_lens
    _say("bf16 decode full llama3_8b (sampled heads)")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, 16, seq, pos)
    dev = _poisoned(plan.num_pages, shape.num_kv_heads, 16)
    kvq.bf16_cache_write(H.to_dev_bf16(k), H.to_dev_bf16(v), H.to_dev(slots), dev)
    q = W.draw_q(shape)
    got = _gpu_decode(shape, plan, dev, q, lens)
    assert np.all(np.isfinite(got))
    # the oracle on two sampled sequences, its cache built from the same tensors
    heads = [(1, 5), (1, 30), (14, 0), (14, 17)]
    for b in sorted({b for b, _ in heads}):
        s1 = shape.with_(batch=1, context_lens=(lens[b],))
        plan1 = W.PagePlan(plan.num_pages, plan.block_table[b:b + 1], plan.capacity[b:b + 1])
        start = int(np.sum(lens[:b]))
        c1 = O.PagedCacheBF16(plan.num_pages, shape.num_kv_heads, 16, 128)
        O.append_bf16(c1, k[start:start + lens[b]], v[start:start + lens[b]], slots[start:start + lens[b]])
        hs = [h for bb, h in heads if bb == b]
        ref = O.decode_bf16(c1, q[b:b + 1], plan1.block_table, np.array([lens[b]]), shape.num_kv_heads,
                            heads=[(0, h) for h in hs])
        for h in hs:
            e = H.rel_l2(got[b, h], ref[0, h])
            assert e <= H.ATTN_RTOL, (b, h, e)

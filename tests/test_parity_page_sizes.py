"""GPU parity at page sizes other than 16 (32, 48, 64: several 16-token tiles per page, and a page
size that is not a power of two for the write path's slot division), for every entry point."""
import numpy as np
import pytest
import torch

import parity_helpers as H
from oracle import kvq_oracle as O
from paged_decode_attention_amd import kvq
from paged_decode_attention_amd import workloads as W
from test_parity_append import compare_caches

pytestmark = pytest.mark.gpu

PAGE_SIZES = [32, 48, 64]


def _say(msg):
    print(msg, flush=True)


def _shape(ps, name="llama3_8b", **kw):
    return W.config(name, batch=3, page_size=ps, **kw).with_(context_lens=(150, 47, 1))


@pytest.mark.parametrize("ps", PAGE_SIZES)
@pytest.mark.parametrize("bits,ts", [(4, 0), (2, 1)])
def test_append_page_sizes(ps, bits, ts):
    shape = _shape(ps, bits=bits, token_scale=ts, hadamard_block=64)
    _say(f"append page size {ps} INT{bits} token_scale {ts}")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, ps, seq, pos)
    ref = O.PagedCache(plan.num_pages, shape.num_kv_heads, ps, 128, bits)
    diag = O.append(ref, k, v, slots, shape.hadamard_block, ts)
    dev = H.poisoned_device_cache(plan.num_pages, shape.num_kv_heads, ps, bits)
    kvq.rotate_quantize_append(H.to_dev_bf16(k), H.to_dev_bf16(v), H.to_dev(slots), dev, shape.hadamard_block, ts)
    torch.cuda.synchronize()
    compare_caches(H.download_cache(dev), ref, [(slots, diag)], f"ps{ps}")


@pytest.mark.parametrize("ps", PAGE_SIZES)
@pytest.mark.parametrize("pps", [0, 1, 1000])
def test_decode_and_step_page_sizes(ps, pps):
    shape = _shape(ps)
    _say(f"decode / decode step / prefill attention, page size {ps}, pages_per_split {pps}")
    lens_prev = shape.context_lens
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, ps, 128, 4)
    O.append(cache, k, v, W.slots_for_positions(plan, ps, seq, pos), shape.hadamard_block, 0)
    dev = H.upload_cache(cache)
    bt = H.to_dev(plan.block_table)
    q = W.draw_q(shape)
    # decode over the prefill
    lens = np.array(lens_prev, dtype=np.int32)
    ref = O.decode(cache, q, plan.block_table, lens, shape.num_kv_heads, shape.hadamard_block)
    got = kvq.paged_decode_attention(H.to_dev_bf16(q), dev, bt, H.to_dev(lens), int(lens.max()), shape.hadamard_block,
                                     pages_per_split=pps)
    torch.cuda.synchronize()
    H.check_attention(got.cpu().numpy(), ref, f"decode ps{ps}")
    # fused decode step: one more token each
    kn, vn = W.draw_kv(shape, shape.batch, stream="decode")
    lens1 = lens + 1
    new_slots = W.slots_for_positions(plan, ps, np.arange(shape.batch), lens)
    d2 = O.append(cache, kn, vn, new_slots, shape.hadamard_block, 0)
    ref1 = O.decode(cache, q, plan.block_table, lens1, shape.num_kv_heads, shape.hadamard_block)
    got1 = kvq.decode_step(H.to_dev_bf16(q), H.to_dev_bf16(kn), H.to_dev_bf16(vn), dev, bt, H.to_dev(lens1),
                           int(lens1.max()), shape.hadamard_block, pages_per_split=pps)
    torch.cuda.synchronize()
    H.check_attention(got1.cpu().numpy(), ref1, f"decode step ps{ps}")
    c_after = H.download_cache(dev)
    k1, v1 = H.cache_codes(c_after)
    k0, v0 = H.cache_codes(cache)
    assert np.mean(k1 != k0) < 1e-4 and np.mean(v1 != v0) < 1e-4   # only boundary codes may differ
    # several queries: the last 3 tokens of each sequence (the one-token sequence has 1)
    q_lens = np.minimum(lens1, 3).astype(np.int32)
    rng = np.random.default_rng(ps)
    qm = W.f32_to_bf16_bits(rng.standard_normal((shape.batch, 3, shape.num_q_heads, 128)).astype(np.float32))
    ref2 = O.multi_query_attention(cache, qm, q_lens, plan.block_table, lens1, shape.num_kv_heads,
                                   shape.hadamard_block)
    got2 = kvq.paged_prefill_attention(H.to_dev_bf16(qm), H.to_dev(q_lens), dev, bt, H.to_dev(lens1),
                                       int(lens1.max()), shape.hadamard_block, pages_per_split=pps)
    torch.cuda.synchronize()
    got2 = got2.cpu().numpy()
    for b in range(shape.batch):
        ql = int(q_lens[b])
        H.check_attention(got2[b, :ql].reshape(-1, 128), ref2[b, :ql].reshape(-1, 128), f"prefill ps{ps} b{b}")
        assert np.all(got2[b, ql:] == 0)


@pytest.mark.parametrize("ps", PAGE_SIZES)
def test_bf16_baseline_page_sizes(ps):
    shape = _shape(ps)
    _say(f"bf16 baseline, page size {ps}")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, ps, seq, pos)
    ref_cache = O.PagedCacheBF16(plan.num_pages, shape.num_kv_heads, ps, 128)
    O.append_bf16(ref_cache, k, v, slots)
    dev = kvq.PagedKVCacheBF16.empty(plan.num_pages, shape.num_kv_heads, ps)
    kvq.bf16_cache_write(H.to_dev_bf16(k), H.to_dev_bf16(v), H.to_dev(slots), dev)
    q = W.draw_q(shape)
    lens = np.array(shape.context_lens, dtype=np.int32)
    ref = O.decode_bf16(ref_cache, q, plan.block_table, lens, shape.num_kv_heads)
    got = kvq.paged_decode_attention_bf16(H.to_dev_bf16(q), dev, H.to_dev(plan.block_table), H.to_dev(lens),
                                          int(lens.max()), pages_per_split=1)
    torch.cuda.synchronize()
    H.check_attention(got.cpu().numpy(), ref, f"bf16 ps{ps}")

"""Seeded random configurations through the write path and the read path, against the oracle.

Each case draws its own shape: 1-5 sequences with ragged prefill lengths (0-400 tokens, some
empty), 1-4 or 8 KV heads, 1-8 query heads per KV head, page size 16, 32, 48 or 64, INT4 or INT2
with or without the per-token scale, a Hadamard block of 1-128 and a split size (the library's
choice, 1, 3 or the whole sequence). The GPU append into a poisoned cache is compared with the
oracle's cache element by element; the GPU decode runs on the oracle's cache, uploaded, with a
NaN-poisoned workspace, and is compared with the oracle's attention for every (sequence, head).
Each case prints its configuration before touching the GPU.
"""
import numpy as np
import pytest
import torch

import parity_helpers as H
from oracle import kvq_oracle as O
from paged_decode_attention_amd import kvq
from paged_decode_attention_amd import workloads as W
from test_parity_append import compare_caches

pytestmark = pytest.mark.gpu

N_CASES = 32


def _say(msg):
    print(msg, flush=True)


def _config(i):
    r = np.random.default_rng(7000 + i)
    kvh = int(r.choice([1, 2, 3, 4, 8]))
    g = int(r.integers(1, 9))
    b = int(r.integers(1, 6))
    lens = [int(n) if r.random() > 0.15 else 0 for n in r.integers(1, 401, size=b)]
    if max(lens) == 0:
        lens[0] = int(r.integers(1, 401))
    ps = int(r.choice([16, 32, 48, 64]))
    bits, ts = [(4, 0), (4, 1), (2, 0), (2, 1)][int(r.integers(0, 4))]
    hb = int(2 ** int(r.integers(0, 8)))
    pps = int(r.choice([0, 0, 1, 3, 1000]))
    shape = W.config("tiny", batch=b, num_q_heads=kvh * g, num_kv_heads=kvh, context_lens=tuple(lens),
                     hadamard_block=hb, bits=bits, token_scale=ts, page_size=ps, seed=7000 + i)
    return shape, pps


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    shape, pps = _config(i)
    ps, hb = shape.page_size, shape.hadamard_block
    _say(f"random case {i}: {shape.batch} seq, lens {shape.context_lens}, heads {shape.num_q_heads}/"
         f"{shape.num_kv_heads}, page {ps}, INT{shape.bits}, token scale {shape.token_scale}, block {hb}, "
         f"pages_per_split {pps}")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, ps, seq, pos)

    # write path
    ref = O.PagedCache(plan.num_pages, shape.num_kv_heads, ps, 128, shape.bits)
    diag = O.append(ref, k, v, slots, hb, shape.token_scale)
    dev = H.poisoned_device_cache(plan.num_pages, shape.num_kv_heads, ps, shape.bits)
    kvq.rotate_quantize_append(H.to_dev_bf16(k), H.to_dev_bf16(v), H.to_dev(slots), dev, hb, shape.token_scale)
    torch.cuda.synchronize()
    compare_caches(H.download_cache(dev), ref, [(slots, diag)], f"case {i}")

    # read path on the oracle's cache
    q = W.draw_q(shape)
    lens = np.array(shape.context_lens, dtype=np.int32)
    max_len = int(lens.max())
    want = O.decode(ref, q, plan.block_table, lens, shape.num_kv_heads, hb)
    nbytes = kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len, ps, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    got = kvq.paged_decode_attention(H.to_dev_bf16(q), H.upload_cache(ref), H.to_dev(plan.block_table),
                                     H.to_dev(lens), max_len, hb, workspace=ws, pages_per_split=pps)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    live = [bb for bb in range(shape.batch) if lens[bb] > 0]
    heads = [(bb, h) for bb in live for h in range(shape.num_q_heads)]
    worst = H.check_attention(got, want, f"case {i}", heads=heads)
    for bb in range(shape.batch):
        if lens[bb] == 0:
            assert np.all(got[bb] == 0), f"case {i}: empty sequence {bb} gives a nonzero output"
    _say(f"  case {i}: worst rel-L2 {worst:.2e}")


def _prefix_cache(shape, lens_prev):
    """The oracle's cache holding each sequence's first lens_prev[b] tokens (room for one more)."""
    s = shape.with_(context_lens=tuple(lens_prev))
    plan = W.plan_pages(s, extra_tokens=1)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, 128, s.bits)
    slots = W.slots_for_positions(plan, s.page_size, seq, pos)
    diag = O.append(cache, k, v, slots, s.hadamard_block, s.token_scale)
    return s, plan, cache, [(slots, diag)]


@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_random_decode_step(i):
    """The fused decode step (append each sequence's newest token, then attend) against the oracle's
    append followed by its decode: the attention and the whole cache afterwards."""
    shape, pps = _config(i)
    lens = np.array(shape.context_lens, dtype=np.int64)  # with the new token
    _say(f"random decode step {i}: lens {tuple(lens)}, heads {shape.num_q_heads}/{shape.num_kv_heads}, "
         f"page {shape.page_size}, INT{shape.bits}, token scale {shape.token_scale}, block {shape.hadamard_block}, "
         f"pages_per_split {pps}")
    s, plan, cache, diags = _prefix_cache(shape, np.maximum(lens - 1, 0))
    dev = H.upload_cache(cache)
    kn, vn = W.draw_kv(s, s.batch, stream="decode")
    live = lens > 0
    new_slots = W.slots_for_positions(plan, s.page_size, np.arange(s.batch), np.maximum(lens - 1, 0))
    new_slots = np.where(live, new_slots, -1).astype(np.int64)
    diags.append((new_slots, O.append(cache, kn, vn, new_slots, s.hadamard_block, s.token_scale)))
    q = W.draw_q(s)
    want = O.decode(cache, q, plan.block_table, lens, s.num_kv_heads, s.hadamard_block)
    max_len = int(lens.max())
    nbytes = kvq.decode_workspace_size(s.batch, s.num_q_heads, s.num_kv_heads, max_len, s.page_size, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    got = kvq.decode_step(H.to_dev_bf16(q), H.to_dev_bf16(kn), H.to_dev_bf16(vn), dev, H.to_dev(plan.block_table),
                          H.to_dev(lens.astype(np.int32)), max_len, s.hadamard_block, token_scale=s.token_scale,
                          workspace=ws, pages_per_split=pps)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    heads = [(bb, h) for bb in range(s.batch) if lens[bb] > 0 for h in range(s.num_q_heads)]
    worst = H.check_attention(got, want, f"step {i}", heads=heads)
    assert all(np.all(got[bb] == 0) for bb in range(s.batch) if lens[bb] == 0), f"step {i}: empty sequence"
    compare_caches(H.download_cache(dev), cache, diags, f"step {i}")
    _say(f"  step {i}: worst rel-L2 {worst:.2e}")


@pytest.mark.parametrize("i", range(N_CASES // 2, N_CASES))
def test_random_multi_query(i):
    """Several queries per sequence (causal, each sequence's last q_lens[b] tokens) against the
    oracle's multi-query attention; rows past a sequence's queries are zero."""
    shape, pps = _config(i)
    r = np.random.default_rng(9000 + i)
    lens = np.array(shape.context_lens, dtype=np.int64)
    q_lens = np.array([int(r.integers(0, min(n, 24) + 1)) for n in lens], dtype=np.int32)
    qmax = max(1, int(q_lens.max()))
    _say(f"random multi-query {i}: lens {tuple(lens)}, q_lens {tuple(q_lens)}, heads {shape.num_q_heads}/"
         f"{shape.num_kv_heads}, page {shape.page_size}, INT{shape.bits}, block {shape.hadamard_block}, "
         f"pages_per_split {pps}")
    s, plan, cache, _ = _prefix_cache(shape, lens)
    q = W.f32_to_bf16_bits(r.standard_normal((s.batch, qmax, s.num_q_heads, 128)).astype(np.float32))
    want = O.multi_query_attention(cache, q, q_lens, plan.block_table, lens, s.num_kv_heads, s.hadamard_block)
    max_len = int(lens.max())
    nbytes = kvq.prefill_workspace_size(s.batch, qmax, s.num_q_heads, s.num_kv_heads, max_len, s.page_size, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    got = kvq.paged_prefill_attention(H.to_dev_bf16(q), H.to_dev(q_lens), H.upload_cache(cache),
                                      H.to_dev(plan.block_table), H.to_dev(lens.astype(np.int32)), max_len,
                                      s.hadamard_block, workspace=ws, pages_per_split=pps)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    rows = [(bb, j, h) for bb in range(s.batch) for j in range(int(q_lens[bb])) for h in range(s.num_q_heads)]
    if rows:
        idx = tuple(np.array(rows).T)
        e = H.rel_l2(got[idx], want[idx])
        assert np.all(np.isfinite(got[idx])) and e.max() <= H.ATTN_RTOL, f"multi-query {i}: worst rel-L2 {e.max():.3e}"
        _say(f"  multi-query {i}: {len(rows)} rows, worst rel-L2 {e.max():.2e}")
    for bb in range(s.batch):
        assert np.all(got[bb, int(q_lens[bb]):] == 0), f"multi-query {i}: rows past sequence {bb}'s queries"

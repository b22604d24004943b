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

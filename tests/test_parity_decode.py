"""GPU parity of kvq_paged_decode_attention and kvq_dequant_page against the CPU oracle.

The cache is always written by the oracle on the host and uploaded, so the read path is
checked on exactly the bytes the oracle attends over. Each case prints its name first.
"""
import math

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


def _oracle_cache(shape, lens, plan=None, layer=0, fast=False):
    s = shape.with_(context_lens=tuple(lens))
    plan = plan or W.plan_pages(s, extra_tokens=0, layer=layer)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq), layer=layer)
    slots = W.slots_for_positions(plan, s.page_size, seq, pos)
    if fast:
        cache, _ = H.host_cache_from_oracle(k, v, slots, plan.num_pages, s.page_size, s.hadamard_block, s.bits,
                                            s.token_scale)
    else:
        cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.bits)
        O.append(cache, k, v, slots, s.hadamard_block, s.token_scale)
    return s, plan, cache


def _gpu_decode(shape, plan, dev_cache, q_bits, lens, pps=0, softmax_scale=0.0, q_prerotated=0):
    max_len = int(max(lens)) if len(lens) else 0
    # the workspace's contents on entry must not matter: poison it with NaN bytes
    nbytes = kvq.decode_workspace_size(len(lens), shape.num_q_heads, shape.num_kv_heads, max_len, shape.page_size, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    out = kvq.paged_decode_attention(
        H.to_dev_bf16(q_bits), dev_cache, H.to_dev(plan.block_table), H.to_dev(np.asarray(lens, dtype=np.int32)),
        max_len, shape.hadamard_block, softmax_scale=softmax_scale, q_prerotated=q_prerotated, workspace=ws,
        pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # name, overrides, lens
    ("tiny", {}, (512,)),
    ("llama3_8b", dict(batch=4), (0, 1, 37, 300)),
    ("llama2_70b", dict(batch=2), (700, 129)),
    ("oscar_int2", dict(batch=3), (500, 16, 250)),
    ("sweep_b8", dict(batch=3), (17, 256, 511)),
]


@pytest.mark.parametrize("name,overrides,lens", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("pps", [0, 1, 2, 1000])
def test_decode_parity(name, overrides, lens, pps):
    shape = W.config(name, **overrides)
    _say(f"decode {name} lens={lens} pages_per_split={pps}")
    s, plan, cache = _oracle_cache(shape, lens)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), s.num_kv_heads, s.hadamard_block)
    got = _gpu_decode(s, plan, H.upload_cache(cache), q, lens, pps=pps)
    worst = H.check_attention(got, ref, f"{name}/pps{pps}")
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)
    _say(f"  worst rel-L2 {worst:.2e}")


@pytest.mark.parametrize("g", [1, 2, 3, 5, 6, 7, 8])
def test_decode_group_sizes(g):
    shape = W.config("llama3_8b", batch=2, num_q_heads=2 * g, num_kv_heads=2, hadamard_block=64)
    lens = (150, 33)
    _say(f"decode GQA group {g}")
    s, plan, cache = _oracle_cache(shape, lens)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), 2, 64)
    H.check_attention(_gpu_decode(s, plan, H.upload_cache(cache), q, lens, pps=3), ref, f"g{g}")


def test_decode_prerotated_query_and_scale():
    shape = W.config("llama3_8b", batch=2)
    lens = (200, 90)
    _say("decode q_prerotated=1, softmax_scale=0.05")
    s, plan, cache = _oracle_cache(shape, lens)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), 8, 128, softmax_scale=0.05, q_prerotated=1)
    got = _gpu_decode(s, plan, H.upload_cache(cache), q, lens, softmax_scale=0.05, q_prerotated=1)
    H.check_attention(got, ref, "prerotated")


def test_decode_page_table_invariance_and_determinism():
    shape = W.config("llama3_8b", batch=2)
    lens = (260, 31)
    _say("decode identity vs shuffled page table; determinism")
    s = shape.with_(context_lens=lens)
    outs = []
    for plan in (W.identity_pages(s, 0), W.plan_pages(s, 0)):
        _, _, cache = _oracle_cache(shape, lens, plan=plan)
        dev = H.upload_cache(cache)
        q = W.draw_q(s)
        a = _gpu_decode(s, plan, dev, q, lens)
        b = _gpu_decode(s, plan, dev, q, lens)
        assert np.array_equal(a, b)
        outs.append(a)
    assert np.array_equal(outs[0], outs[1])


def test_decode_split_invariance():
    """Split counts 1 (auto here), many and few give the same attention: each meets the oracle
    bound, and they agree with each other to 1e-3. They are not bit-identical: every split runs its
    own online softmax against its own running maximum, so p * delta - fed to the matrix cores as a
    bf16 hi + lo pair (about 2^-17 relative rounding) - rounds differently per split."""
    shape = W.config("llama2_70b", batch=1)
    lens = (2000,)
    _say("decode split invariance")
    s, plan, cache = _oracle_cache(shape, lens)
    dev = H.upload_cache(cache)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), s.num_kv_heads, s.hadamard_block)
    outs = [_gpu_decode(s, plan, dev, q, lens, pps=p) for p in (0, 1, 7, 125)]
    for p, o in zip((0, 1, 7, 125), outs):
        H.check_attention(o, ref, f"pps{p}")
    for o in outs[1:]:
        assert np.all(H.rel_l2(o, outs[0]) < 1e-3)


@pytest.mark.parametrize("lens,pps", [((384, 100, 17, 250), 1), ((272, 100, 17, 250), 1), ((256, 33, 1, 200), 1),
                                      ((640, 100, 17, 250), 2), ((1024, 64, 3, 512), 4)])
def test_decode_split_groups(lens, pps):
    """Sequences in 16 or more splits run four splits to a workgroup and combine them in LDS: 24, 17,
    16, 20 and 16 splits of the longest sequence (17 leaves a group whose waves past the last split
    have no pages), and the shorter sequences leave waves and whole groups empty (rows with maximum
    -inf in the combine and the merge)."""
    shape = W.config("llama3_8b", batch=4, hadamard_block=64)
    _say(f"decode split groups lens={lens} pages_per_split={pps}")
    s, plan, cache = _oracle_cache(shape, lens)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), s.num_kv_heads, s.hadamard_block)
    got = _gpu_decode(s, plan, H.upload_cache(cache), q, lens, pps=pps)
    H.check_attention(got, ref, f"split groups {lens} pps{pps}")
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


def test_decode_side_stream_own_workspace():
    """Calls on a side stream that pass no workspace: the wrapper allocates each call's split
    workspace with that stream current, so the memory it frees at return cannot be handed to work
    on another stream while the call may still run. The current stream allocates and fills fresh
    memory right after every call; every result equals the same call made on the current stream."""
    shape = W.config("llama3_8b", batch=2)
    lens = (900, 400)
    _say("decode on a side stream with the wrapper's own workspace")
    s, plan, cache = _oracle_cache(shape, lens)
    dev = H.upload_cache(cache)
    q = H.to_dev_bf16(W.draw_q(s))
    bt, ln = H.to_dev(plan.block_table), H.to_dev(np.asarray(lens, dtype=np.int32))
    assert kvq.decode_workspace_size(2, s.num_q_heads, s.num_kv_heads, 900, 16, 4) > 0
    ref = kvq.paged_decode_attention(q, dev, bt, ln, 900, s.hadamard_block, pages_per_split=4)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    outs = [torch.empty_like(ref) for _ in range(6)]
    junk = []
    for o in outs:
        kvq.paged_decode_attention(q, dev, bt, ln, 900, s.hadamard_block, out=o, pages_per_split=4, stream=side)
        junk.append(torch.full((1 << 20,), 0xFF, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref), f"side-stream call {i} differs from the current-stream call"


@pytest.mark.parametrize("tensor", ["k", "v"])
@pytest.mark.parametrize("bits,ts,hb", [(4, 0, 32), (2, 1, 128), (4, 0, 1)])
def test_dequant_page(tensor, bits, ts, hb):
    shape = W.config("tiny", batch=1, num_q_heads=4, num_kv_heads=4, context_lens=(40,), bits=bits, token_scale=ts,
                     hadamard_block=hb)
    _say(f"dequant page {tensor} int{bits} hb={hb}")
    s, plan, cache = _oracle_cache(shape, (40,))
    dev = H.upload_cache(cache)
    for page in (int(plan.block_table[0, 0]), int(plan.block_table[0, 2])):
        for un in (0, 1):
            got = kvq.dequant_page(dev, tensor, page, hb, unrotate=un).cpu().numpy()
            ref = O.dequant_page(cache, page, hb, un, tensor=tensor)
            torch.cuda.synchronize()
            live = ~np.isnan(ref[:, :, 0])
            if un == 0:
                # one fused multiply-add: the correctly rounded value of code * scale + zero
                assert np.array_equal(got[live], ref[live])
            else:
                err = np.abs(got[live].astype(np.float64) - ref[live])
                mag = np.abs(ref[live]).max(axis=-1, keepdims=True)
                assert np.all(err <= 1e-6 * mag + 1e-30)


# ----------------------------------------------------------------------------- full sizes

def _full_size_sampled(name, n_samples, layer=0, longest=False):
    """The whole workload in one launch (the library's split plan, as the benchmark runs it); every
    query head of n_samples sampled (sequence, KV head) items compared with the oracle (the oracle
    gathers an item's sequence once, so the whole group costs no more than one head)."""
    shape = W.config(name)
    lens = shape.context_lens
    _say(f"decode full {name} lens={lens[0]}..{max(lens)}x{len(lens)} (sampled items)")
    s, plan, cache = _oracle_cache(shape, lens, layer=layer, fast=True)
    q = W.draw_q(s, layer=layer)
    got = _gpu_decode(s, plan, H.upload_cache(cache), q, lens)
    assert np.all(np.isfinite(got))
    g = s.num_q_heads // s.num_kv_heads
    rng = np.random.default_rng(99)
    items = {(int(b), int(kvh)) for b, kvh in zip(rng.integers(0, s.batch, n_samples),
                                                  rng.integers(0, s.num_kv_heads, n_samples))}
    if longest:  # the sequence with the most splits, every KV head
        b_max = int(np.argmax(lens))
        items |= {(b_max, kvh) for kvh in range(s.num_kv_heads)}
    heads = sorted((b, kvh * g + j) for b, kvh in items for j in range(g))
    ref = O.decode(cache, q, plan.block_table, np.array(lens), s.num_kv_heads, s.hadamard_block, heads=heads)
    worst = H.check_attention(got, ref, f"full {name}", heads=heads)
    _say(f"  {len(items)} sampled items, {len(heads)} heads, worst rel-L2 {worst:.2e}")


def test_decode_full_llama3_8b():
    _full_size_sampled("llama3_8b", 12)


def test_decode_full_llama2_70b_one_layer():
    _full_size_sampled("llama2_70b", 6)


def test_decode_full_oscar_int2():
    _full_size_sampled("oscar_int2", 8)


def test_decode_full_sweep_b32():
    # 32 ragged sequences x 8 KV heads fill the waves with few splits per sequence, so the planned
    # splits are capped at 48 pages (the longest sequence, 7407 tokens, takes 10)
    _full_size_sampled("sweep_b32", 8, longest=True)

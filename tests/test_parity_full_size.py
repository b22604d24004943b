"""GPU parity at the benchmark's full sizes, in the launch configurations the benchmark times.

- The fused decode step on the whole Llama-3-8B-shaped layer (16 sequences x 4096 cached tokens
  + the new one, 32/8 heads, the library's split plan): every query head of five whole
  (sequence, KV head) items against the oracle - each item spans all its splits, among them the
  one that holds the page with the new token - and the whole cache afterwards, including the 16 x 8
  rows the step wrote.
- Decode attention at batch 256 of the concurrency sweep (1.1 M ragged tokens): the oracle
  caches four whole sequences (the longest, the shortest and two others), the GPU runs the full
  launch, and every query head of those sequences is compared.
- The OScaR INT2 chunked prefill (32 x 16384 tokens, 512-token chunks landing mid-page) through
  the GPU append, call by call as the benchmark issues it, against the oracle's placement of
  every token: the whole cache, byte by byte.
- The attention of a 512-token chunk over the OScaR cache (32 x 16384 tokens, 28/4 heads, every
  sequence with 512 queries: the large-chunk kernel's full grid): the oracle caches three whole
  sequences, and every head of ten query rows of each (the first two, the middle one, the last
  two and five more) is compared; the whole output must be finite.

Each case prints its name before it touches the GPU.
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


def _say(msg):
    print(msg, flush=True)


def _t_diag(diag):
    """compare_caches' view of a host_cache_from_oracle diagnosis (the pre-rounding values)."""
    return {"k_t": diag["k"][3], "v_t": diag["v"][3]}


def _item_heads(items, g):
    return sorted((b, kvh * g + j) for b, kvh in items for j in range(g))


@pytest.mark.timeout(600)
def test_decode_step_full_llama3_8b():
    shape = W.config("llama3_8b")
    ps, hb, ts = shape.page_size, shape.hadamard_block, shape.token_scale
    _say("decode step full llama3_8b: 16 x (4096 + 1) tokens, 32/8 heads, library split plan")
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, ps, seq, pos)
    cache, d1 = H.host_cache_from_oracle(k, v, slots, plan.num_pages, ps, hb, shape.bits, ts)
    del k, v
    dev = H.upload_cache(cache)
    dseq, dpos = W.decode_positions(shape)
    kn, vn = W.draw_kv(shape, shape.batch, stream="decode")
    new_slots = W.slots_for_positions(plan, ps, dseq, dpos)
    d2 = O.append(cache, kn, vn, new_slots, hb, ts)
    lens = np.asarray(shape.context_lens, dtype=np.int32) + 1
    max_len = int(lens.max())
    q = W.draw_q(shape)
    g = shape.num_q_heads // shape.num_kv_heads
    items = [(0, 0), (3, 7), (8, 2), (12, 5), (15, 3)]
    heads = _item_heads(items, g)
    ref = O.decode(cache, q, plan.block_table, lens, shape.num_kv_heads, hb, heads=heads)
    nbytes = kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len, ps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    out = kvq.decode_step(H.to_dev_bf16(q), H.to_dev_bf16(kn), H.to_dev_bf16(vn), dev, H.to_dev(plan.block_table),
                          H.to_dev(lens), max_len, hb, token_scale=ts, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite attention output"
    worst = H.check_attention(got, ref, "decode step full llama3_8b", heads=heads)
    _say(f"  {len(items)} items x {g} heads, worst rel-L2 {worst:.2e}")
    compare_caches(H.download_cache(dev), cache, [(slots, _t_diag(d1)), (new_slots, d2)],
                   "decode step full llama3_8b cache")


@pytest.mark.timeout(600)
def test_decode_full_sweep_b256():
    shape = W.config("sweep_b256")
    ps, hb = shape.page_size, shape.hadamard_block
    lens = np.asarray(shape.context_lens, dtype=np.int64)
    rng = np.random.default_rng(256)
    picked = sorted({int(np.argmax(lens)), int(np.argmin(lens)), *(int(x) for x in rng.integers(0, shape.batch, 2))})
    _say(f"decode full sweep_b256: {int(lens.sum())} tokens; oracle sequences {picked} "
         f"(lengths {[int(lens[b]) for b in picked]})")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    keep = np.isin(seq, picked)
    k, v = W.draw_kv(shape, int(keep.sum()))
    slots = W.slots_for_positions(plan, ps, seq[keep], pos[keep])
    cache, _ = H.host_cache_from_oracle(k, v, slots, plan.num_pages, ps, hb, shape.bits, shape.token_scale)
    del k, v
    # the other sequences' pages hold zero scale and zero: finite outputs that nothing checks
    for a in (cache.k_sz, cache.v_sz):
        a[np.isnan(a)] = 0.0
    q = W.draw_q(shape)
    g = shape.num_q_heads // shape.num_kv_heads
    heads = _item_heads([(b, kvh) for b in picked for kvh in range(shape.num_kv_heads)], g)
    ref = O.decode(cache, q, plan.block_table, lens, shape.num_kv_heads, hb, heads=heads)
    max_len = int(lens.max())
    nbytes = kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max_len, ps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    out = kvq.paged_decode_attention(H.to_dev_bf16(q), H.upload_cache(cache), H.to_dev(plan.block_table),
                                     H.to_dev(lens.astype(np.int32)), max_len, hb, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite attention output"
    worst = H.check_attention(got, ref, "decode full sweep_b256", heads=heads)
    _say(f"  {len(picked)} sequences x {shape.num_q_heads} heads, worst rel-L2 {worst:.2e}")


@pytest.mark.timeout(900)
def test_append_full_oscar_chunked_prefill():
    shape = W.config("oscar_int2")
    ps, hb, ts = shape.page_size, shape.hadamard_block, shape.token_scale
    plan = W.plan_pages(shape, extra_tokens=1)
    calls = W.chunk_schedule(shape)
    n_tok = sum(len(sq) for sq, _ in calls)
    _say(f"append full oscar_int2 chunked prefill: {len(calls)} calls, {n_tok} tokens x {shape.num_kv_heads} heads")
    k, v = W.draw_kv(shape, n_tok)
    slot_list = [W.slots_for_positions(plan, ps, sq, pp) for sq, pp in calls]
    dev = H.poisoned_device_cache(plan.num_pages, shape.num_kv_heads, ps, shape.bits)
    k_d, v_d = H.to_dev_bf16(k), H.to_dev_bf16(v)
    o = 0
    for sl in slot_list:
        kvq.rotate_quantize_append(k_d[o:o + len(sl)], v_d[o:o + len(sl)], H.to_dev(sl), dev, hb, ts)
        o += len(sl)
    torch.cuda.synchronize()
    del k_d, v_d
    got = H.download_cache(dev)
    del dev
    slots = np.concatenate(slot_list)
    ref, diag = H.host_cache_from_oracle(k, v, slots, plan.num_pages, ps, hb, shape.bits, ts)
    compare_caches(got, ref, [(slots, _t_diag(diag))], "oscar_int2 chunked prefill")


@pytest.mark.timeout(600)
def test_chunk_attention_full_oscar():
    shape = W.config("oscar_int2")
    ps, hb = shape.page_size, shape.hadamard_block
    lens = np.asarray(shape.context_lens, dtype=np.int64)
    qmax = shape.chunk
    picked = [0, 13, 31]
    assert kvq.prefill_kernel(shape.batch, qmax, shape.num_q_heads, shape.num_kv_heads) == 1
    _say(f"chunk attention full oscar_int2: {shape.batch} x {qmax} queries x {shape.num_q_heads} heads over "
         f"{int(lens.max())} tokens; oracle sequences {picked}")
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    keep = np.isin(seq, picked)
    k, v = W.draw_kv(shape, int(keep.sum()))
    slots = W.slots_for_positions(plan, ps, seq[keep], pos[keep])
    cache, _ = H.host_cache_from_oracle(k, v, slots, plan.num_pages, ps, hb, shape.bits, shape.token_scale)
    del k, v
    # the other sequences' pages hold zero scale and zero: finite outputs that nothing checks
    for a in (cache.k_sz, cache.v_sz):
        a[np.isnan(a)] = 0.0
    rng = np.random.default_rng(shape.seed + 77)
    q = W.f32_to_bf16_bits(rng.standard_normal((shape.batch, qmax, shape.num_q_heads, 128), dtype=np.float32))
    r = np.random.default_rng(5120)
    js = sorted({0, 1, qmax // 2, qmax - 2, qmax - 1, *r.choice(qmax, 5, replace=False).tolist()})
    rows = [(b, j, h) for b in picked for h in range(shape.num_q_heads) for j in js]  # one gather per KV head
    q_lens = np.full(shape.batch, qmax, dtype=np.int32)
    ref = O.multi_query_attention(cache, q, q_lens, plan.block_table, lens, shape.num_kv_heads, hb, rows=rows)
    out = kvq.paged_prefill_attention(H.to_dev_bf16(q), H.to_dev(q_lens), H.upload_cache(cache),
                                      H.to_dev(plan.block_table), H.to_dev(lens.astype(np.int32)), int(lens.max()),
                                      hb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite attention output"
    worst = 0.0
    for b in picked:
        worst = max(worst, H.check_attention(got[b, js].reshape(-1, 128), ref[b, js].reshape(-1, 128),
                                             f"chunk attention full oscar_int2 b{b}"))
    _say(f"  {len(rows)} rows, worst rel-L2 {worst:.2e}")

"""GPU parity of kvq_paged_prefill_attention on large chunks - at least 128 (query, head) columns
per KV head and 256 blocks of them, where the library dequantizes each cache tile once per 256
columns into LDS (fp16 operands on the matrix cores) - against the oracle's multi-query
attention: every query row of every sequence in the fixed cases, sampled rows in the seeded
random ones.

The shapes cover INT4 and INT2 (per-token scaling), GQA 4, 7 and 8, page sizes 16, 32 and 64,
ragged contexts whose last tile ends mid-tile (the rows past each sequence hold the oracle
cache's NaN poison), queries per sequence from 0 to the maximum, and a last workgroup that is
only partly filled with columns.
"""
import dataclasses

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


def _case(name, overrides, lens):
    shape = W.config(name, **overrides).with_(context_lens=tuple(lens))
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
    O.append(cache, k, v, W.slots_for_positions(plan, shape.page_size, seq, pos), shape.hadamard_block,
             shape.token_scale)
    return shape, plan, cache


def _queries(shape, qmax, seed):
    rng = np.random.default_rng(seed)
    return W.f32_to_bf16_bits(rng.standard_normal((shape.batch, qmax, shape.num_q_heads, 128)).astype(np.float32))


def _gpu(shape, plan, dev, q, q_lens, lens, q_prerotated=0, softmax_scale=0.0, workspace=True):
    qmax = q.shape[1]
    max_len = int(max(lens))
    nbytes = kvq.prefill_workspace_size(shape.batch, qmax, shape.num_q_heads, shape.num_kv_heads, max_len,
                                        shape.page_size)
    # (the large-chunk kernel leaves it untouched: without one the binding passes a null workspace)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda") if workspace else None
    out = torch.full((shape.batch, qmax, shape.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    kvq.paged_prefill_attention(H.to_dev_bf16(q), H.to_dev(np.asarray(q_lens, dtype=np.int32)), dev,
                                H.to_dev(plan.block_table), H.to_dev(np.asarray(lens, dtype=np.int32)), max_len,
                                shape.hadamard_block, softmax_scale=softmax_scale, out=out, workspace=ws,
                                q_prerotated=q_prerotated)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # name, overrides, context lens, q_lens, max_q_len
    ("oscar_int2", dict(batch=3), (700, 600, 520), (512, 300, 513), 513),                     # INT2, g 7
    ("llama3_8b", dict(batch=4), (300, 1000, 256, 700), (256, 100, 0, 37), 256),              # INT4, g 4
    ("llama2_70b", dict(batch=2, page_size=32), (450, 333), (256, 200), 256),                 # g 8, pages of 32
    ("llama3_8b", dict(batch=4, page_size=64, hadamard_block=16), (129, 640, 300, 77), (129, 64, 256, 77), 256),
]


@pytest.mark.parametrize("name,overrides,lens,q_lens,qmax", CASES,
                         ids=[f"{c[0]}-ps{c[1].get('page_size', 16)}" for c in CASES])
def test_chunk_attention_parity(name, overrides, lens, q_lens, qmax):
    shape, plan, cache = _case(name, overrides, lens)
    assert kvq.prefill_kernel(shape.batch, qmax, shape.num_q_heads, shape.num_kv_heads) == 1, "not a large-chunk launch"
    _say(f"chunk attention {name} {overrides} lens={lens} q_lens={q_lens}")
    q = _queries(shape, qmax, seed=sum(lens) + qmax)
    ref = O.multi_query_attention(cache, q, np.array(q_lens), plan.block_table, np.array(lens), shape.num_kv_heads,
                                  shape.hadamard_block)
    got = _gpu(shape, plan, H.upload_cache(cache), q, q_lens, lens)
    assert np.all(np.isfinite(got))
    for b, ql in enumerate(q_lens):
        ql = min(ql, lens[b])
        assert np.all(got[b, ql:] == 0), f"rows past q_lens[{b}] must be zero"
        if ql:
            worst = H.check_attention(got[b, :ql].reshape(-1, 128), ref[b, :ql].reshape(-1, 128), f"{name}/b{b}")
            _say(f"  b{b}: {ql} queries, worst rel-L2 {worst:.2e}")


def test_chunk_attention_prerotated_query():
    """q_prerotated = 1 with R q given equals q_prerotated = 0 with q (same launch shape); called
    with no workspace (a null pointer through the C ABI)."""
    shape, plan, cache = _case("llama3_8b", dict(batch=4), (300, 280, 256, 400))
    assert kvq.prefill_kernel(4, 256, 32, 8) == 1
    q_lens = (256, 256, 256, 256)
    q = _queries(shape, 256, seed=11)
    r = O.rotation_matrix(128, shape.hadamard_block)
    qr = W.f32_to_bf16_bits((W.bf16_bits_to_f32(q).astype(np.float64) @ r.T).astype(np.float32))
    _say("chunk attention, prerotated query")
    dev = H.upload_cache(cache)
    ref = O.multi_query_attention(cache, qr, np.array(q_lens), plan.block_table, np.array((300, 280, 256, 400)),
                                  shape.num_kv_heads, shape.hadamard_block, q_prerotated=1)
    got = _gpu(shape, plan, dev, qr, q_lens, (300, 280, 256, 400), q_prerotated=1, workspace=False)
    worst = H.check_attention(got.reshape(-1, 128), ref.reshape(-1, 128), "prerotated")
    _say(f"  worst rel-L2 {worst:.2e}")


def test_chunk_attention_cache_scales():
    """The same cache with every V (or K) scale and zero multiplied by 2^-40 or 2^40 - values far
    outside fp16's range: the output scales by exactly that power of two for V, and does not change
    for K when the softmax scale undoes it, so the tiles' power-of-two exponents carry the range."""
    lens = (300, 513, 256, 77)
    shape, plan, cache = _case("llama3_8b", dict(batch=4), lens)
    assert kvq.prefill_kernel(4, 256, 32, 8) == 1
    q_lens = (256, 256, 256, 77)
    q = _queries(shape, 256, seed=12)
    base = _gpu(shape, plan, H.upload_cache(cache), q, q_lens, lens)
    for tensor in ("v", "k"):
        for e in (-40, 40):
            scaled = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
            for name in ("k_codes", "v_codes", "k_sz", "v_sz"):
                setattr(scaled, name, getattr(cache, name).copy())
            sz = getattr(cache, f"{tensor}_sz")
            setattr(scaled, f"{tensor}_sz", (sz.astype(np.float64) * 2.0 ** e).astype(np.float32))
            _say(f"chunk attention, {tensor.upper()} scale and zero x 2^{e}")
            sm = 2.0 ** -e / np.sqrt(128.0) if tensor == "k" else 0.0
            got = _gpu(shape, plan, H.upload_cache(scaled), q, q_lens, lens, softmax_scale=sm)
            want = base.astype(np.float64) * (2.0 ** e if tensor == "v" else 1.0)
            worst = 0.0
            for b, ql in enumerate(q_lens):
                assert np.all(got[b, ql:] == 0)
                worst = max(worst, H.check_attention(got[b, :ql].reshape(-1, 128), want[b, :ql].reshape(-1, 128),
                                                     f"{tensor} x 2^{e}"))
            _say(f"  worst rel-L2 against the unscaled output {worst:.2e}")


def _random_config(i):
    r = np.random.default_rng(9100 + i)
    kvh = int(r.choice([4, 8]))
    g = int(r.integers(1, 5))
    qmax = int(r.choice([128, 160, 256]))
    per_seq = -(-qmax * g // 128) * kvh                  # workgroups per sequence
    b = max(2, -(-256 // per_seq))                        # at least 256 workgroups in all
    q_lens = [int(x) for x in r.integers(1, qmax + 1, size=b)]
    q_lens[0] = qmax
    if b > 2:
        q_lens[1] = 0                                     # a sequence without queries
    lens = [ql + int(r.integers(0, 300)) for ql in q_lens]
    lens[1] = max(lens[1], 1)
    ps = int(r.choice([16, 32, 64]))
    bits, ts = [(4, 0), (4, 1), (2, 0), (2, 1)][int(r.integers(0, 4))]
    hb = int(2 ** int(r.integers(0, 8)))
    shape = W.config("tiny", batch=b, num_q_heads=kvh * g, num_kv_heads=kvh, context_lens=tuple(lens),
                     hadamard_block=hb, bits=bits, token_scale=ts, page_size=ps, seed=9100 + i)
    return shape, q_lens, qmax


@pytest.mark.parametrize("i", range(6))
def test_chunk_attention_random(i):
    """Seeded random large-chunk configurations: 4 or 8 KV heads, GQA 1-4, 128-256 queries per
    sequence (ragged, one sequence without any), contexts up to 300 tokens past the queries, pages
    of 16/32/64, INT4/INT2 with and without the token scale, Hadamard blocks 1-128; the whole
    output is checked for finiteness and zero padding, sampled query rows against the oracle."""
    shape, q_lens, qmax = _random_config(i)
    assert kvq.prefill_kernel(shape.batch, qmax, shape.num_q_heads, shape.num_kv_heads) == 1
    lens = shape.context_lens
    _say(f"chunk random {i}: {shape.batch} seq, lens {lens}, q_lens {q_lens}, heads {shape.num_q_heads}/"
         f"{shape.num_kv_heads}, page {shape.page_size}, INT{shape.bits}, token scale {shape.token_scale}, "
         f"block {shape.hadamard_block}")
    plan = W.plan_pages(shape, extra_tokens=0)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
    O.append(cache, k, v, W.slots_for_positions(plan, shape.page_size, seq, pos), shape.hadamard_block,
             shape.token_scale)
    q = _queries(shape, qmax, seed=9100 + i)
    # Sampled query rows (every head of each): the first two and last two of each sequence, its
    # middle one and up to 20 more at random.
    r = np.random.default_rng(9200 + i)
    picks = {b: sorted({0, 1, ql // 2, ql - 2, ql - 1, *r.choice(ql, size=min(ql, 20), replace=False).tolist()}
                       & set(range(ql))) for b, ql in enumerate(q_lens) if ql}
    rows = [(b, j, h) for b, js in picks.items() for h in range(shape.num_q_heads) for j in js]  # one gather per head
    ref = O.multi_query_attention(cache, q, np.array(q_lens), plan.block_table, np.array(lens), shape.num_kv_heads,
                                  shape.hadamard_block, rows=rows)
    got = _gpu(shape, plan, H.upload_cache(cache), q, q_lens, lens)
    assert np.all(np.isfinite(got))
    worst = 0.0
    for b, ql in enumerate(q_lens):
        assert np.all(got[b, ql:] == 0)
        if ql:
            js = picks[b]
            worst = max(worst, H.check_attention(got[b, js].reshape(-1, 128), ref[b, js].reshape(-1, 128),
                                                 f"random {i} b{b}"))
    _say(f"  worst rel-L2 over {len(rows)} sampled rows {worst:.2e}")


def test_chunk_attention_skips_invalid_pages():
    """Page-table entries outside [0, num_pages) are skipped: the attention equals the oracle's over
    the sequence with those pages' tokens left out (built from the oracle's gather and attend)."""
    lens = (300, 600, 280, 400)
    shape, plan, cache = _case("llama3_8b", dict(batch=4), lens)
    q_lens = (256, 256, 256, 200)
    assert kvq.prefill_kernel(4, 256, 32, 8) == 1
    bt = plan.block_table.copy()
    dropped = {0: [3, 7], 1: [1, 20, 30]}                 # (sequence: page indices) made invalid
    for b, pages in dropped.items():
        for j, p in enumerate(pages):
            bt[b, p] = -1 if j % 2 == 0 else plan.num_pages + 5
    q = _queries(shape, 256, seed=13)
    _say("chunk attention with invalid page ids")
    got = _gpu(shape, dataclasses.replace(plan, block_table=bt), H.upload_cache(cache), q, q_lens, lens)
    assert np.all(np.isfinite(got))
    g = shape.group
    r = O.rotation_matrix(128, shape.hadamard_block)
    scale = 1.0 / np.sqrt(128.0)
    rng = np.random.default_rng(3)
    for b in (0, 1, 2):
        ps = shape.page_size
        keep = np.ones(lens[b], dtype=bool)
        for p in dropped.get(b, []):
            keep[p * ps:(p + 1) * ps] = False
        for kvh in range(shape.num_kv_heads):
            kh, vh = O.gather_sequence(cache, plan.block_table[b], lens[b], kvh)
            for j in sorted(rng.choice(q_lens[b], 24, replace=False)):
                n = lens[b] - q_lens[b] + j + 1
                sel = keep[:n]
                for hh in range(g):
                    h = kvh * g + hh
                    qq = r @ O.bf16_to_f32(q[b, j, h]).astype(np.float64)
                    want = r.T @ O.attend(qq, kh[:n][sel], vh[:n][sel], scale)
                    e = H.rel_l2(got[b, j, h], want)
                    assert e <= H.ATTN_RTOL, (b, j, h, float(e))

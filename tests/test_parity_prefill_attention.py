"""GPU parity of kvq_paged_prefill_attention (several queries per sequence, causal: chunked
prefill and speculative verification) against the oracle's multi-query attention."""
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


def _case(name, overrides, lens, layer=0):
    shape = W.config(name, **overrides).with_(context_lens=tuple(lens))
    plan = W.plan_pages(shape, extra_tokens=0, layer=layer)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq), layer=layer)
    cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
    O.append(cache, k, v, W.slots_for_positions(plan, shape.page_size, seq, pos), shape.hadamard_block,
             shape.token_scale)
    return shape, plan, cache


def _queries(shape, qmax, seed):
    rng = np.random.default_rng(seed)
    return W.f32_to_bf16_bits(rng.standard_normal((shape.batch, qmax, shape.num_q_heads, 128)).astype(np.float32))


def _gpu(shape, plan, dev, q, q_lens, lens, pps=0):
    qmax = q.shape[1]
    max_len = int(max(lens))
    nbytes = kvq.prefill_workspace_size(shape.batch, qmax, shape.num_q_heads, shape.num_kv_heads, max_len,
                                        shape.page_size, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    out = kvq.paged_prefill_attention(H.to_dev_bf16(q), H.to_dev(np.asarray(q_lens, dtype=np.int32)), dev,
                                      H.to_dev(plan.block_table), H.to_dev(np.asarray(lens, dtype=np.int32)), max_len,
                                      shape.hadamard_block, workspace=ws, pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # name, overrides, context lens, q_lens, max_q_len
    ("tiny", {}, (512,), (16,), 16),                                         # g = 1: 16 queries, one tile
    ("llama3_8b", dict(batch=3), (300, 77, 16), (4, 2, 4), 4),               # speculative: 4 x 4 heads = 16 columns
    ("llama2_70b", dict(batch=2), (700, 129), (5, 0), 5),                    # g = 8: 40 columns, a partial tile
    ("oscar_int2", dict(batch=2), (600, 100), (64, 37), 64),                 # chunk of 64, g = 7, INT2 + token scale
    ("sweep_b8", dict(batch=2, hadamard_block=1), (45, 300), (45, 9), 48),   # a whole sequence as its own chunk
]


@pytest.mark.parametrize("name,overrides,lens,q_lens,qmax", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("pps", [0, 1, 1000])
def test_prefill_attention_parity(name, overrides, lens, q_lens, qmax, pps):
    _say(f"prefill attention {name} lens={lens} q_lens={q_lens} pages_per_split={pps}")
    shape, plan, cache = _case(name, overrides, lens)
    q = _queries(shape, qmax, seed=len(lens) * 100 + qmax)
    ref = O.multi_query_attention(cache, q, np.array(q_lens), plan.block_table, np.array(lens), shape.num_kv_heads,
                                  shape.hadamard_block)
    got = _gpu(shape, plan, H.upload_cache(cache), q, q_lens, lens, pps)
    assert np.all(np.isfinite(got))
    for b, ql in enumerate(q_lens):
        assert np.all(got[b, ql:] == 0)
        if ql:
            worst = H.check_attention(got[b, :ql].reshape(-1, 128), ref[b, :ql].reshape(-1, 128), f"{name}/b{b}")
            _say(f"  b{b}: worst rel-L2 {worst:.2e}")


def test_prefill_attention_one_query_is_decode():
    """max_q_len = 1 with q_lens = 1 gives the decode's attention (same kernel family, same plan)."""
    shape, plan, cache = _case("llama3_8b", dict(batch=3), (300, 77, 16))
    _say("prefill attention with one query vs decode")
    dev = H.upload_cache(cache)
    q = W.draw_q(shape)
    lens = np.array([300, 77, 16], dtype=np.int32)
    got = _gpu(shape, plan, dev, q[:, None], [1, 1, 1], lens)[:, 0]
    dec = kvq.paged_decode_attention(H.to_dev_bf16(q), dev, H.to_dev(plan.block_table), H.to_dev(lens), 300,
                                     shape.hadamard_block).cpu().numpy()
    assert np.all(H.rel_l2(got, dec) < 1e-3)


def test_prefill_attention_chunk_512_sampled():
    """A 512-token chunk at the end of 2 x 2048-token Llama-3-8B-shaped sequences, sampled rows."""
    shape, plan, cache = _case("llama3_8b", dict(batch=2), (2048, 1500))
    _say("prefill attention, 512-token chunk (sampled rows)")
    q = _queries(shape, 512, seed=7)
    q_lens = (512, 300)
    got = _gpu(shape, plan, H.upload_cache(cache), q, q_lens, (2048, 1500))
    rng = np.random.default_rng(5)
    rows = sorted({(int(b), int(j), int(h)) for b, j, h in
                   zip(rng.integers(0, 2, 24), rng.integers(0, 512, 24), rng.integers(0, 32, 24))})
    ref = O.multi_query_attention(cache, q, np.array(q_lens), plan.block_table, np.array([2048, 1500]), 8, 128,
                                  rows=rows)
    for b, j, h in rows:
        if j >= q_lens[b]:
            assert np.all(got[b, j, h] == 0)
        else:
            e = H.rel_l2(got[b, j, h], ref[b, j, h])
            assert e <= H.ATTN_RTOL, (b, j, h, e)

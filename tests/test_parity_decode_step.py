"""GPU parity of the fused decode step (kvq_decode_step: append each sequence's new token at
position L - 1, then attend over L tokens) against the oracle's append followed by its decode:
the attention output and the whole cache after the call."""
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


CASES = [
    ("tiny", {}, (512,)),
    ("llama3_8b", dict(batch=4), (1, 17, 300, 0)),
    ("llama2_70b", dict(batch=2), (700, 129)),
    ("oscar_int2", dict(batch=3), (500, 16, 33)),
    ("sweep_b8", dict(batch=3, hadamard_block=1), (64, 65, 2)),
]


@pytest.mark.parametrize("name,overrides,lens", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("pps", [0, 1, 1000])
def test_decode_step_parity(name, overrides, lens, pps):
    shape = W.config(name, **overrides)
    _say(f"decode step {name} lens (with the new token)={lens} pages_per_split={pps}")
    prev = tuple(max(n - 1, 0) for n in lens)
    s = shape.with_(context_lens=prev)
    plan = W.plan_pages(s, extra_tokens=1)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.bits)
    d1 = O.append(cache, k, v, W.slots_for_positions(plan, s.page_size, seq, pos), s.hadamard_block, s.token_scale)
    dev = H.upload_cache(cache)
    # the new tokens (one per sequence; none where L = 0)
    kn, vn = W.draw_kv(s, s.batch, stream="decode")
    live = np.array([n > 0 for n in lens])
    new_slots = W.slots_for_positions(plan, s.page_size, np.arange(s.batch), np.maximum(np.array(lens) - 1, 0))
    new_slots = np.where(live, new_slots, -1).astype(np.int64)
    d2 = O.append(cache, kn, vn, new_slots, s.hadamard_block, s.token_scale)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), s.num_kv_heads, s.hadamard_block)
    max_len = int(max(lens))
    nbytes = kvq.decode_workspace_size(s.batch, s.num_q_heads, s.num_kv_heads, max_len, s.page_size, pps)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    out = kvq.decode_step(H.to_dev_bf16(q), H.to_dev_bf16(kn), H.to_dev_bf16(vn), dev, H.to_dev(plan.block_table),
                          H.to_dev(np.asarray(lens, dtype=np.int32)), max_len, s.hadamard_block,
                          token_scale=s.token_scale, workspace=ws, pages_per_split=pps)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = H.check_attention(got, ref, f"step {name}/pps{pps}")
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)
    diags = [(W.slots_for_positions(plan, s.page_size, seq, pos), d1), (new_slots, d2)]
    compare_caches(H.download_cache(dev), cache, diags, f"step {name}/pps{pps}")
    _say(f"  worst rel-L2 {worst:.2e}")


@pytest.mark.parametrize("bits,ts", [(4, 0), (2, 1)])
def test_decode_step_extreme_new_tokens(bits, ts):
    """New tokens whose RMS and scale lie far outside [2^-100, 2^101) (tiny, about 1e-33, and huge,
    about 1e31, normal values) take the fused quantizer's guarded division; the cache rows and the
    attention still match the oracle's append followed by its decode."""
    shape = W.config("llama3_8b", batch=4, bits=bits, token_scale=ts)
    lens = (40, 17, 100, 64)
    _say(f"decode step extreme new tokens INT{bits} token scale {ts}")
    prev = tuple(n - 1 for n in lens)
    s = shape.with_(context_lens=prev)
    plan = W.plan_pages(s, extra_tokens=1)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.bits)
    d1 = O.append(cache, k, v, W.slots_for_positions(plan, s.page_size, seq, pos), s.hadamard_block, s.token_scale)
    dev = H.upload_cache(cache)
    r = np.random.default_rng(31)
    mags = np.array([1e-33, 1e31, 1e-33, 1.0])[:, None, None]
    kn = W.f32_to_bf16_bits((r.standard_normal((4, s.num_kv_heads, 128)) * mags).astype(np.float32))
    vn = W.f32_to_bf16_bits((r.standard_normal((4, s.num_kv_heads, 128)) * mags[::-1]).astype(np.float32))
    new_slots = W.slots_for_positions(plan, s.page_size, np.arange(4), np.array(lens) - 1).astype(np.int64)
    d2 = O.append(cache, kn, vn, new_slots, s.hadamard_block, s.token_scale)
    q = W.draw_q(s)
    ref = O.decode(cache, q, plan.block_table, np.array(lens), s.num_kv_heads, s.hadamard_block)
    max_len = max(lens)
    out = kvq.decode_step(H.to_dev_bf16(q), H.to_dev_bf16(kn), H.to_dev_bf16(vn), dev, H.to_dev(plan.block_table),
                          H.to_dev(np.asarray(lens, dtype=np.int32)), max_len, s.hadamard_block,
                          token_scale=s.token_scale)
    torch.cuda.synchronize()
    H.check_attention(out.cpu().numpy(), ref, f"extreme INT{bits}")
    compare_caches(H.download_cache(dev), cache, [(W.slots_for_positions(plan, s.page_size, seq, pos), d1),
                                                  (new_slots, d2)], f"extreme INT{bits}")


def test_decode_step_matches_separate_calls():
    """One fused launch and the two separate calls (append, then attention) leave the same cache
    and the same attention within the attention tolerance."""
    shape = W.config("llama3_8b", batch=3)
    lens = (200, 33, 16)
    _say("decode step vs separate append + attention")
    prev = tuple(n - 1 for n in lens)
    s = shape.with_(context_lens=prev)
    plan = W.plan_pages(s, extra_tokens=1)
    seq, pos = W.prefill_order(s)
    k, v = W.draw_kv(s, len(seq))
    cache = O.PagedCache(plan.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.bits)
    O.append(cache, k, v, W.slots_for_positions(plan, s.page_size, seq, pos), s.hadamard_block, 0)
    kn, vn = W.draw_kv(s, s.batch, stream="decode")
    q = H.to_dev_bf16(W.draw_q(s))
    bt, lens_d = H.to_dev(plan.block_table), H.to_dev(np.asarray(lens, dtype=np.int32))
    fused, separate = H.upload_cache(cache), H.upload_cache(cache)
    o1 = kvq.decode_step(q, H.to_dev_bf16(kn), H.to_dev_bf16(vn), fused, bt, lens_d, max(lens), s.hadamard_block)
    new_slots = W.slots_for_positions(plan, 16, np.arange(3), np.array(lens) - 1)
    kvq.rotate_quantize_append(H.to_dev_bf16(kn), H.to_dev_bf16(vn), H.to_dev(new_slots), separate, s.hadamard_block)
    o2 = kvq.paged_decode_attention(q, separate, bt, lens_d, max(lens), s.hadamard_block)
    torch.cuda.synchronize()
    assert np.all(H.rel_l2(o1.cpu().numpy(), o2.cpu().numpy()) < 1e-3)
    c1, c2 = H.download_cache(fused), H.download_cache(separate)
    # the two write paths round the rotation differently (butterfly vs matrix cores): codes may differ
    # by one step at rounding boundaries only
    k1, v1 = H.cache_codes(c1)
    k2, v2 = H.cache_codes(c2)
    assert np.abs(k1.astype(int) - k2.astype(int)).max() <= 1 and np.abs(v1.astype(int) - v2.astype(int)).max() <= 1
    assert (k1 != k2).mean() < 1e-4 and (v1 != v2).mean() < 1e-4

"""kvq_paged_decode_attention_noalloc: the decode with its split partials in the library's fixed
scratch. Through the C ABI it must give what kvq_paged_decode_attention gives with a caller
workspace (the same kernels: bit for bit), and both must meet the oracle's attention bound; two
calls in a row, the second smaller, share the scratch. Sizes whose partials exceed the scratch
are refused before any launch."""
import numpy as np
import pytest
import torch

import parity_helpers as H
from oracle import kvq_oracle as O
from paged_decode_attention_amd import kvq
from paged_decode_attention_amd import workloads as W


def _say(msg):
    print(msg, flush=True)


def test_oversized_partials_are_refused_before_launch():
    """Host only: the status comes back before anything touches the device (stand-in pointers)."""
    L = kvq.lib()
    p = 1 << 12  # aligned, never dereferenced

    def call(b, hq, hkv, mcl, pps, mpps):
        return L.kvq_paged_decode_attention_noalloc(p, 0, p, p, p, p, 1 << 20, 16, p, mpps, p, mcl, b, hq, hkv, 128,
                                                    128, 4, 0.0, p, pps, None)
    # 33 splits of 16 pages x 256 sequences x 32 heads x 520 bytes (140 MB): far beyond 16 MiB
    need = kvq.decode_workspace_size(256, 32, 8, 8193, 16, 16)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    assert call(256, 32, 8, 8193, 16, 513) == kvq.KVQ_ERR_WORKSPACE
    # other argument errors keep their own status
    assert call(256, 30, 8, 8193, 16, 513) == kvq.KVQ_ERR_SHAPE
    assert call(0, 32, 8, 8193, 16, 513) == kvq.KVQ_OK


CALLS = [
    # name, overrides, lens, pages_per_split: the second call is smaller than the first
    ("llama3_8b", dict(batch=4), (700, 1500, 33, 2049), 16),
    ("llama3_8b", dict(batch=2), (300, 17), 4),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_twice():
    for i, (name, over, lens, pps) in enumerate(CALLS):
        shape = W.config(name, **over).with_(context_lens=tuple(lens))
        need = kvq.decode_workspace_size(shape.batch, shape.num_q_heads, shape.num_kv_heads, max(lens),
                                         shape.page_size, pps)
        _say(f"no-alloc call {i}: {name} lens {lens} pages_per_split {pps} partial bytes {need}")
        assert 0 < need <= kvq.NOALLOC_SCRATCH_BYTES
        plan = W.plan_pages(shape, extra_tokens=0)
        seq, pos = W.prefill_order(shape)
        k, v = W.draw_kv(shape, len(seq))
        cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
        O.append(cache, k, v, W.slots_for_positions(plan, shape.page_size, seq, pos), shape.hadamard_block,
                 shape.token_scale)
        q = W.draw_q(shape)
        want = O.decode(cache, q, plan.block_table, np.asarray(lens), shape.num_kv_heads, shape.hadamard_block)
        dev = H.upload_cache(cache)
        q_d, bt, lens_d = H.to_dev_bf16(q), H.to_dev(plan.block_table), H.to_dev(np.asarray(lens, dtype=np.int32))
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        ref = kvq.paged_decode_attention(q_d, dev, bt, lens_d, max(lens), shape.hadamard_block, workspace=ws,
                                         pages_per_split=pps)
        out = torch.full_like(ref, float("nan"))
        got = kvq.paged_decode_attention_noalloc(q_d, dev, bt, lens_d, max(lens), shape.hadamard_block, out,
                                                 pages_per_split=pps)
        torch.cuda.synchronize()
        got, ref = got.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref), f"call {i}: the two entry points differ"
        worst = H.check_attention(got, want, f"no-alloc call {i}")
        _say(f"  call {i}: identical to the workspace decode, worst rel-L2 against the oracle {worst:.2e}")

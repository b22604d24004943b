"""The entry points inside a captured HIP graph: each replay (with eager work and synchronisations
between replays) must give the eager result bit for bit. The launches take the caller's stream,
allocate nothing and clear nothing with memset, so a caller may capture them."""
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


def test_append_and_decode_replayed_from_a_graph():
    shape = W.config("llama3_8b", batch=3).with_(context_lens=(700, 33, 300))
    _say("graph capture: append + split decode + fused step, 3 replays")
    plan = W.plan_pages(shape, extra_tokens=1)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = H.to_dev(W.slots_for_positions(plan, 16, seq, pos).astype(np.int64))
    kd, vd = H.to_dev_bf16(k), H.to_dev_bf16(v)
    q = H.to_dev_bf16(W.draw_q(shape))
    bt = H.to_dev(plan.block_table)
    lens = np.array(shape.context_lens, dtype=np.int32)
    lens_d = H.to_dev(lens)
    max_len = int(lens.max())
    kn, vn = (H.to_dev_bf16(x) for x in W.draw_kv(shape, shape.batch, stream="decode"))
    lens1_d = H.to_dev(lens + 1)
    ws = kvq.decode_workspace(kvq.decode_workspace_size(shape.batch, 32, 8, max_len + 1, 16, 2), "cuda")

    def work(cache, out, out1):
        kvq.rotate_quantize_append(kd, vd, slots, cache, 128, 0)
        kvq.paged_decode_attention(q, cache, bt, lens_d, max_len, 128, out=out, workspace=ws, pages_per_split=2)
        kvq.decode_step(q, kn, vn, cache, bt, lens1_d, max_len + 1, 128, out=out1, workspace=ws, pages_per_split=2)

    # eager reference
    ref_cache = H.poisoned_device_cache(plan.num_pages, 8, 16, 4)
    ref_out = torch.empty((shape.batch, 32, 128), dtype=torch.float32, device="cuda")
    ref_out1 = torch.empty_like(ref_out)
    work(ref_cache, ref_out, ref_out1)
    torch.cuda.synchronize()
    # captured
    cache = H.poisoned_device_cache(plan.num_pages, 8, 16, 4)
    out = torch.empty_like(ref_out)
    out1 = torch.empty_like(ref_out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(cache, out, out1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(cache, out, out1)
    for r in range(3):
        # eager work between replays: a fresh cache written and read on the default stream
        for c in (cache,):
            for t in (c.k_codes, c.v_codes):
                t.fill_(0xAA)
            for t in (c.k_sz, c.v_sz):
                t.fill_(float("nan"))
        out.fill_(float("nan"))
        out1.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("k_codes", "v_codes", "k_sz", "v_sz"):
            a, b = getattr(cache, name), getattr(ref_cache, name)
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r}: {name} differs"
        assert torch.equal(out, ref_out), f"replay {r}: decode output differs"
        assert torch.equal(out1, ref_out1), f"replay {r}: fused step output differs"
        extra = kvq.paged_decode_attention(q, ref_cache, bt, lens_d, max_len, 128)   # eager, own buffers
        torch.cuda.synchronize()
        assert torch.isfinite(extra).all()
    # and the eager reference itself matches the oracle
    host = O.PagedCache(plan.num_pages, 8, 16, 128, 4)
    O.append(host, k, v, W.slots_for_positions(plan, 16, seq, pos), 128, 0)
    want = O.decode(host, W.draw_q(shape), plan.block_table, lens, 8, 128)
    H.check_attention(ref_out.cpu().numpy(), want, "graph reference")

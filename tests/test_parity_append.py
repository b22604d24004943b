"""GPU parity of kvq_rotate_quantize_append against the CPU oracle.

Each case prints its name, seed and shape before touching the GPU. Caches start poisoned
(0xAA code bytes, NaN scale/zero), so a stray or missing write shows up as a byte that does
not match the oracle's (identically poisoned) cache.
"""
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


def _gpu_append(k_bits, v_bits, slots, num_pages, kv_heads, bits, hb, ts, dev_cache=None, stride_pad=0):
    cache = dev_cache or H.poisoned_device_cache(num_pages, kv_heads, 16, bits)
    if stride_pad:
        t_n = k_bits.shape[0]
        big_k = torch.zeros((t_n, kv_heads + stride_pad, 128), dtype=torch.bfloat16, device="cuda")
        big_v = torch.zeros((t_n, kv_heads + 2 * stride_pad, 128), dtype=torch.bfloat16, device="cuda")
        big_k[:, :kv_heads] = H.to_dev_bf16(k_bits)
        big_v[:, :kv_heads] = H.to_dev_bf16(v_bits)
        k_dev, v_dev = big_k[:, :kv_heads], big_v[:, :kv_heads]
    else:
        k_dev, v_dev = H.to_dev_bf16(k_bits), H.to_dev_bf16(v_bits)
    kvq.rotate_quantize_append(k_dev, v_dev, H.to_dev(slots.astype(np.int64)), cache, hb, ts)
    torch.cuda.synchronize()
    return cache


def compare_caches(got: O.PagedCache, ref: O.PagedCache, diags, what):
    """Whole-cache comparison. ``diags``: list of (slots, diag) from the oracle appends, in order."""
    bits = ref.bits
    # every byte of every untouched row is still poison in both
    written = ~np.isnan(ref.k_sz[..., 0])                     # [P, H, ps]
    assert np.array_equal(np.isnan(got.k_sz[..., 0]), ~written), f"{what}: K rows written that the oracle did not write (or missed)"
    assert np.array_equal(np.isnan(got.v_sz[..., 0]), ~written), f"{what}: V rows written/missed"
    gk, gv = H.cache_codes(got)
    rk, rv = H.cache_codes(ref)
    p, h, ps = written.shape
    kraw_g = got.k_codes[~written]
    assert np.all(kraw_g == 0xAA), f"{what}: K bytes changed in unwritten rows"
    vraw_g = got.v_codes.transpose(0, 1, 2, 4, 3).reshape(p, h, ps, -1)[~written]
    assert np.all(vraw_g == 0xAA), f"{what}: V bytes changed in unwritten rows"
    # codes of written rows: exact except boundary elements, with t from the last write of each slot
    t_k = np.zeros(rk.shape, dtype=np.float64)
    t_v = np.zeros(rv.shape, dtype=np.float64)
    for slots, d in diags:
        live = (slots >= 0) & (slots < p * ps)
        pg, of = slots[live] // ps, slots[live] % ps
        for hh in range(h):
            t_k[pg, hh, of] = d["k_t"][live, hh]
            t_v[pg, hh, of] = d["v_t"][live, hh]
    nk = H.check_codes(gk[written], rk[written], t_k[written], f"{what} K")
    nv = H.check_codes(gv[written], rv[written], t_v[written], f"{what} V")
    H.check_scale_zero(got.k_sz[written][:, 0], got.k_sz[written][:, 1], ref.k_sz[written][:, 0],
                       ref.k_sz[written][:, 1], bits, f"{what} K")
    H.check_scale_zero(got.v_sz[written][:, 0], got.v_sz[written][:, 1], ref.v_sz[written][:, 0],
                       ref.v_sz[written][:, 1], bits, f"{what} V")
    _say(f"  {what}: {written.sum()} rows, boundary mismatches K {nk} V {nv}")
    return nk + nv


def _prefill_case(shape, layer=0):
    plan = W.plan_pages(shape, layer=layer)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq), layer=layer)
    slots = W.slots_for_positions(plan, shape.page_size, seq, pos)
    return plan, k, v, slots


@pytest.mark.parametrize("name,overrides", [
    ("tiny", {}),
    ("llama3_8b", dict(batch=2, context_lens=(300, 77))),
    ("sweep_b8", dict(batch=3, context_lens=(513, 64, 1))),
    ("llama2_70b", dict(batch=1, context_lens=(333,))),
])
def test_append_prefill(name, overrides):
    shape = W.config(name, **overrides)
    _say(f"append prefill {name} {overrides} seed {shape.seed}")
    plan, k, v, slots = _prefill_case(shape)
    got = H.download_cache(_gpu_append(k, v, slots, plan.num_pages, shape.num_kv_heads, shape.bits,
                                       shape.hadamard_block, shape.token_scale))
    ref = O.PagedCache(plan.num_pages, shape.num_kv_heads, 16, 128, shape.bits)
    d = O.append(ref, k, v, slots, shape.hadamard_block, shape.token_scale)
    compare_caches(got, ref, [(slots, d)], name)


@pytest.mark.parametrize("hb", [1, 2, 4, 8, 16, 32, 64, 128])
@pytest.mark.parametrize("bits,ts", [(4, 0), (2, 1), (4, 1), (2, 0)])
def test_append_block_sizes(hb, bits, ts):
    shape = W.config("tiny", batch=2, num_q_heads=4, num_kv_heads=4, context_lens=(45, 20), hadamard_block=hb,
                     bits=bits, token_scale=ts, lognorm_sigma=2.0)
    _say(f"append hb={hb} bits={bits} ts={ts}")
    plan, k, v, slots = _prefill_case(shape)
    got = H.download_cache(_gpu_append(k, v, slots, plan.num_pages, 4, bits, hb, ts))
    ref = O.PagedCache(plan.num_pages, 4, 16, 128, bits)
    d = O.append(ref, k, v, slots, hb, ts)
    compare_caches(got, ref, [(slots, d)], f"hb{hb}/int{bits}/ts{ts}")


def test_append_chunked_int2_partial_pages():
    """OScaR-style INT2 with per-token scaling; chunks start inside partially filled pages."""
    shape = W.config("oscar_int2", batch=3, context_lens=(600, 130, 45), chunk=128)
    _say(f"append chunked INT2 {shape.context_lens}")
    plan = W.plan_pages(shape)
    dev = H.poisoned_device_cache(plan.num_pages, shape.num_kv_heads, 16, 2)
    ref = O.PagedCache(plan.num_pages, shape.num_kv_heads, 16, 128, 2)
    diags = []
    for ci, (seq, pos) in enumerate(W.chunk_schedule(shape)):
        k, v = W.draw_kv(shape, len(seq), layer=ci)
        slots = W.slots_for_positions(plan, 16, seq, pos)
        _gpu_append(k, v, slots, plan.num_pages, shape.num_kv_heads, 2, 128, 1, dev_cache=dev)
        diags.append((slots, O.append(ref, k, v, slots, 128, 1)))
    compare_caches(H.download_cache(dev), ref, diags, "chunked INT2")


def test_append_skips_strides_and_degenerate_tokens():
    shape = W.config("tiny", batch=1, num_q_heads=8, num_kv_heads=8, context_lens=(70,))
    _say("append skips / strides / degenerate tokens")
    plan, k, v, slots = _prefill_case(shape)
    slots = slots.copy()
    slots[[0, 5, 33]] = -1                                  # padding tokens
    slots[[7]] = plan.num_pages * 16 + 3                   # beyond the pool: ignored
    k = k.copy()
    v = v.copy()
    k[10] = 0                                              # all-zero vectors (scale 0, and RMS 0)
    v[11] = W.f32_to_bf16_bits(np.full((8, 128), 3.5, dtype=np.float32))   # constant vectors
    k[12, :, 0] = W.f32_to_bf16_bits(np.full(8, 3.0e4, dtype=np.float32))  # one huge outlier
    # tokens whose RMS and scale lie far outside [2^-100, 2^101): tiny (about 1e-33) and huge (about
    # 1e31) normal values, which take the division's guarded path
    r = np.random.default_rng(13)
    k[13] = W.f32_to_bf16_bits((r.standard_normal((8, 128)) * 1e-33).astype(np.float32))
    v[14] = W.f32_to_bf16_bits((r.standard_normal((8, 128)) * 1e31).astype(np.float32))
    for bits, ts in ((4, 0), (2, 1)):
        got = H.download_cache(_gpu_append(k, v, slots, plan.num_pages, 8, bits, 32, ts, stride_pad=3))
        ref = O.PagedCache(plan.num_pages, 8, 16, 128, bits)
        d = O.append(ref, k, v, np.where(slots < plan.num_pages * 16, slots, -1), 32, ts)
        compare_caches(got, ref, [(np.where(slots < plan.num_pages * 16, slots, -1), d)], f"edge int{bits}")


def test_append_zero_tokens_and_determinism():
    shape = W.config("tiny", context_lens=(100,))
    _say("append zero tokens / determinism")
    plan, k, v, slots = _prefill_case(shape)
    dev = H.poisoned_device_cache(plan.num_pages, 8, 16, 4)
    kvq.rotate_quantize_append(H.to_dev_bf16(k[:0]), H.to_dev_bf16(v[:0]), H.to_dev(slots[:0]), dev, 32)
    torch.cuda.synchronize()
    assert torch.all(dev.k_codes == 0xAA) and torch.all(torch.isnan(dev.k_sz))
    a = H.download_cache(_gpu_append(k, v, slots, plan.num_pages, 8, 4, 32, 0))
    b = H.download_cache(_gpu_append(k, v, slots, plan.num_pages, 8, 4, 32, 0))
    assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.v_codes, b.v_codes)
    assert np.array_equal(a.k_sz, b.k_sz, equal_nan=True) and np.array_equal(a.v_sz, b.v_sz, equal_nan=True)


def test_append_full_llama3_8b_prefill():
    """The full Llama-3-8B-shaped prefill (16 x 4096 tokens x 8 KV heads) in the launch
    configuration the benchmark times; every row compared."""
    shape = W.config("llama3_8b")
    _say("append full llama3_8b prefill 16x4096x8")
    plan, k, v, slots = _prefill_case(shape)
    dev = _gpu_append(k, v, slots, plan.num_pages, 8, 4, 128, 0)
    got = H.download_cache(dev)
    del dev
    ref, diag = H.host_cache_from_oracle(k, v, slots, plan.num_pages, 16, 128, 4, 0)
    live = slots >= 0
    pg, of = slots // 16, slots % 16
    gk, gv = H.cache_codes(got)
    n_bad = 0
    for name, gc, sz in (("k", gk, got.k_sz), ("v", gv, got.v_sz)):
        cq, sc, zr, t = diag[name]
        g_codes = gc[pg, :, of, :]                            # [T, H, D]
        n_bad += H.check_codes(g_codes, cq, t, f"full {name}")
        H.check_scale_zero(sz[pg, :, of, 0], sz[pg, :, of, 1], sc, zr, 4, f"full {name}")
    assert np.array_equal(np.isnan(got.k_sz), np.isnan(ref.k_sz))
    _say(f"  full prefill: {live.sum() * 8 * 2 * 128} elements, boundary mismatches {n_bad}")


@pytest.mark.parametrize("bits", [4, 2])
def test_append_rounding_ties_exact(bits):
    """Codes that fall exactly halfway between two integers round to the even one, on the GPU as in
    the oracle, with no boundary allowance. With a Hadamard block of 1 the rotation is the identity,
    and a token whose values span exactly [o, o + qmax] * 2^e has the scale 2^e and the zero o * 2^e,
    so (y - zero) / scale is the token's pattern value itself: the expected codes are rint of the
    pattern (half to even), a closed form independent of the oracle."""
    qmax = 2 ** bits - 1
    rng = np.random.default_rng(31 + bits)
    t_n, h_n = 32, 2
    ties = [k + 0.5 for k in range(qmax)]
    base = np.array([0.0, float(qmax)] + ties, dtype=np.float64)
    quarters = rng.integers(0, 4 * qmax + 1, size=(t_n, h_n, 2, 128 - base.size)) / 4.0
    pattern = np.concatenate([np.broadcast_to(base, (t_n, h_n, 2, base.size)), quarters], axis=-1)
    pattern = np.take_along_axis(pattern, rng.permuted(np.tile(np.arange(128), (t_n, h_n, 2, 1)), axis=-1), axis=-1)
    offset = rng.choice([0.0, -8.0, 3.5, -0.25, 6.0], size=(t_n, h_n, 2, 1))
    e = rng.integers(-3, 4, size=(t_n, h_n, 2, 1)).astype(np.float64)
    values = (pattern + offset) * 2.0 ** e
    bits16 = W.f32_to_bf16_bits(values.astype(np.float32))
    back = (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, values), "pattern values must be exact in bf16"
    k, v = np.ascontiguousarray(bits16[:, :, 0]), np.ascontiguousarray(bits16[:, :, 1])
    slots = np.arange(t_n, dtype=np.int64)
    _say(f"rounding ties INT{bits}: {t_n} tokens x {h_n} heads, Hadamard block 1")
    got = H.download_cache(_gpu_append(k, v, slots, 2, h_n, bits, 1, 0))
    ref = O.PagedCache(2, h_n, 16, 128, bits)
    O.append(ref, k, v, slots, 1, 0)
    gk, gv = H.cache_codes(got)
    rk, rv = H.cache_codes(ref)
    want = np.rint(pattern).astype(np.uint8)                      # numpy rounds half to even
    assert np.all(want[np.isin(pattern, ties)] % 2 == 0)
    for name, g, r, j in (("K", gk, rk, 0), ("V", gv, rv, 1)):
        g = g.transpose(0, 2, 1, 3).reshape(t_n, h_n, 128)         # [P, H, ps, D] -> [T, H, D]
        r = r.transpose(0, 2, 1, 3).reshape(t_n, h_n, 128)
        assert np.array_equal(r, want[:, :, j]), f"oracle {name} codes differ from the closed form"
        assert np.array_equal(g, want[:, :, j]), f"GPU {name} codes differ from the closed form"
    for sz, j in ((got.k_sz, 0), (got.v_sz, 1)):
        s = sz.transpose(0, 2, 1, 3).reshape(t_n, h_n, 2)
        assert np.array_equal(s[..., 0].astype(np.float64), (2.0 ** e[:, :, j, 0])), "scale is not 2^e"
        assert np.array_equal(s[..., 1].astype(np.float64), offset[:, :, j, 0] * 2.0 ** e[:, :, j, 0]), "zero is not o 2^e"

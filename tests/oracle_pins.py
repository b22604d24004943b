"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a closed form,
a library routine, a hand-derived golden value, an invariant or a brute-force computation.
They are plain functions (not collected by pytest on their own) so that
``test_oracle_pins.py`` runs them on the real oracle and ``test_oracle_mutations.py`` runs
them on copies of the oracle with planted mistakes, to show each mistake is caught.

The oracle module is looked up at call time (``O.name``), so a test that patches an
attribute of ``oracle.kvq_oracle`` is seen by every pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import kvq_oracle as O
from paged_decode_attention_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)


def _bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------------------- Hadamard

def pin_hadamard_orthogonal():
    for n in (1, 2, 4, 8, 16, 32, 64, 128):
        h = O.hadamard(n)
        assert set(np.unique(h)) <= {-1, 1}
        assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64)), n


def pin_hadamard_scipy():
    import scipy.linalg
    for n in (2, 4, 8, 16, 32, 64, 128):
        assert np.array_equal(O.hadamard(n), scipy.linalg.hadamard(n)), n


def pin_hadamard_golden_h8():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "hadamard_sylvester_8.txt")) if ln.strip() and not ln.startswith("#")]
    h8 = np.array(rows, dtype=np.int64)
    assert np.array_equal(O.hadamard(8), h8)


def pin_hadamard_doubling():
    h = np.array([[1]], dtype=np.int64)
    for n in (2, 4, 8, 16, 32, 64, 128):
        h = np.block([[h, h], [h, -h]])
        assert np.array_equal(O.hadamard(n), h), n


def pin_rotation_orthonormal():
    for b in (1, 2, 4, 8, 16, 32, 64, 128):
        r = O.rotation_matrix(128, b)
        assert np.array_equal(r, r.T)
        assert np.abs(r @ r - np.eye(128)).max() < 1e-14
        # block structure: zero outside the diagonal blocks
        mask = np.kron(np.eye(128 // b), np.ones((b, b))) == 0
        assert np.all(r[mask] == 0)
    assert np.array_equal(O.rotation_matrix(128, 1), np.eye(128))


def _fwht_reference(x: np.ndarray, b: int) -> np.ndarray:
    """Textbook in-place fast Walsh-Hadamard butterflies (float32), one block at a time."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    for s in range(0, d, b):
        blk = y[..., s:s + b]
        h = 1
        while h < b:
            for i in range(0, b, 2 * h):
                a = blk[..., i:i + h].copy()
                c = blk[..., i + h:i + 2 * h].copy()
                blk[..., i:i + h] = a + c
                blk[..., i + h:i + 2 * h] = a - c
            h *= 2
        y[..., s:s + b] = blk
    return y * np.float32(1.0 / math.sqrt(b))


def pin_rotation_fwht():
    rng = np.random.default_rng(5)
    for b in (1, 2, 4, 8, 16, 32, 64, 128):
        xi = rng.integers(-8, 9, size=(16, 128)).astype(np.float32)      # small integers: every sum exact
        assert np.array_equal(O.rotate_f32(xi, b), _fwht_reference(xi, b)), b
        xr = W.bf16_bits_to_f32(_bits(rng.standard_normal((64, 128)) * 3))
        got, ref = O.rotate_f32(xr, b), _fwht_reference(xr, b)
        tol = 4 * np.finfo(np.float32).eps * np.abs(xr).sum(axis=-1, keepdims=True)
        assert np.all(np.abs(got - ref) <= tol), b


def pin_rotation_golden():
    for ex in _golden()["rotation"]:
        b, x = ex["b"], np.array([ex["x"]], dtype=np.float32)
        y = O.rotate_f32(x, b)[0]
        if "y" in ex:
            assert np.array_equal(y, np.array(ex["y"], dtype=np.float32)), ex
        else:
            want = np.array(ex["y_over_inv_sqrt_b"], dtype=np.float32) * np.float32(1.0 / math.sqrt(b))
            assert np.array_equal(y, want), ex


def pin_rotation_constant_vector():
    for b in (2, 4, 8, 16, 32, 64, 128):
        for c in (1.0, -3.0, 0.375):
            y = O.rotate_f32(np.full((1, 128), c, dtype=np.float32), b)[0].astype(np.float64)
            want = np.zeros(128)
            want[::b] = c * math.sqrt(b)
            assert np.allclose(y, want, rtol=1e-6, atol=0), (b, c)


def pin_rotation_invariants():
    rng = np.random.default_rng(11)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128) * 5
    for b in (1, 2, 8, 32, 64, 128):
        r = O.rotation_matrix(128, b)
        assert abs(np.linalg.norm(r @ k) - np.linalg.norm(k)) < 1e-12 * np.linalg.norm(k)
        assert abs((r @ q) @ (r @ k) - q @ k) < 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)
        # the float32 path preserves norms to float32 accuracy
        x = W.bf16_bits_to_f32(_bits(k))
        y = O.rotate_f32(x[None, :], b)[0].astype(np.float64)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x.astype(np.float64))) < 1e-6 * np.linalg.norm(x)


# ----------------------------------------------------------------------------- quantizer

def pin_quantizer_golden():
    g = _golden()
    for ex in g["quantize"]:
        u = np.array([ex["u"]], dtype=np.float32)
        codes, scale, zero, _ = O.quantize_rows(u, ex["bits"])
        assert np.array_equal(codes[0], np.array(ex["codes"], dtype=np.uint8)), ex
        assert scale[0] == np.float32(ex["scale"]) and zero[0] == np.float32(ex["zero"]), ex
    for ex in g["token_scale"]:
        x = _bits(ex["y"])
        assert np.array_equal(W.bf16_bits_to_f32(x), np.array(ex["y"], dtype=np.float32))
        codes, scale, zero, _ = O.rotate_quantize(x[None, :], ex["b"], ex["bits"], 1)
        assert np.array_equal(codes[0], np.array(ex["codes"], dtype=np.uint8)), ex
        assert abs(scale[0] - ex["scale"]) <= 1e-6 * abs(ex["scale"])
        assert abs(zero[0] - ex["zero"]) <= 1e-6 * max(abs(ex["zero"]), ex["scale"])


def pin_quantizer_error_bound():
    rng = np.random.default_rng(3)
    for bits in (2, 4):
        u = (rng.standard_normal((2000, 128)) * rng.lognormal(0, 1.5, size=(2000, 1))).astype(np.float32)
        codes, scale, zero, _ = O.quantize_rows(u, bits)
        qmax = 2 ** bits - 1
        assert codes.max() <= qmax
        deq = codes.astype(np.float64) * scale[:, None] + zero[:, None]
        ulp = np.spacing(np.abs(u).max(axis=1, keepdims=True)).astype(np.float64)
        assert np.all(np.abs(deq - u) <= scale[:, None] / 2 + 4 * ulp)
        # extremes land exactly on 0 and qmax
        assert np.all(codes[np.arange(len(u)), u.argmin(axis=1)] == 0)
        assert np.all(codes[np.arange(len(u)), u.argmax(axis=1)] == qmax)
        # zero is the minimum, scale the range over qmax
        assert np.array_equal(zero, u.min(axis=1))
        assert np.array_equal(scale, (u.max(axis=1) - u.min(axis=1)) / np.float32(qmax))
        # mean squared error of uniform rounding: scale^2 / 12 (within 10 %)
        err = ((deq - u) / scale[:, None]) ** 2
        inner = (codes > 0) & (codes < qmax)
        assert abs(err[inner].mean() - 1 / 12) < 0.1 / 12


def pin_quantizer_grid_and_affine():
    rng = np.random.default_rng(4)
    for bits in (2, 4):
        qmax = 2 ** bits - 1
        c = rng.integers(0, qmax + 1, size=(100, 128))
        c[:, 0], c[:, 1] = 0, qmax
        for a, off in ((0.25, 3.0), (2.0, -7.0), (1.0 / 64, 0.5)):
            u = (c * a + off).astype(np.float32)
            codes, scale, zero, _ = O.quantize_rows(u, bits)
            assert np.array_equal(codes, c.astype(np.uint8))
            assert np.all(scale == np.float32(a)) and np.all(zero == np.float32(off))
        # affine invariance for power-of-two gains (every float32 step exact)
        u = rng.standard_normal((100, 128)).astype(np.float32)
        c0 = O.quantize_rows(u, bits)[0]
        for a in (0.125, 4.0, 1024.0):
            assert np.array_equal(O.quantize_rows(u * np.float32(a), bits)[0], c0)


def pin_quantizer_degenerate():
    u = np.zeros((3, 128), dtype=np.float32)
    u[1] = 2.5
    u[2] = -1e-3
    codes, scale, zero, _ = O.quantize_rows(u, 4)
    assert np.all(codes == 0) and np.all(scale == 0)
    assert np.array_equal(zero, u[:, 0])
    # the per-token scaling step must not produce NaN on an all-zero token
    c2, s2, z2, _ = O.rotate_quantize(np.zeros((1, 128), dtype=np.uint16), 128, 2, 1)
    assert np.all(c2 == 0) and s2[0] == 0 and z2[0] == 0


def pin_token_rms_closed_form():
    """The per-token scale is the root mean square: +-a entries give exactly a, a 3-4-5 vector
    padded with zeros gives sqrt(25 / d), an all-zero token gives 1, and the result is the
    float32 rounding of the float64 value (not a float32 running sum)."""
    d = 128
    signs = np.where(np.arange(d) % 3 == 0, -1.0, 1.0).astype(np.float32)
    y = np.stack([signs * np.float32(0.375), np.zeros(d, np.float32), np.zeros(d, np.float32)])
    y[2, 0], y[2, 1] = 3.0, 4.0
    s = O.token_rms(y)
    assert s[0] == np.float32(0.375)
    assert s[1] == np.float32(1.0)
    assert s[2] == np.float32(math.sqrt(25.0 / d))
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((64, d)) * 1e3).astype(np.float32)
    want = np.sqrt(np.sum(z.astype(np.float64) ** 2, axis=1) / d).astype(np.float32)
    assert np.array_equal(O.token_rms(z), want)


def pin_token_scale_fold():
    """Per-token scaling folds into scale/zero: codes equal those of the unscaled path except
    at rounding boundaries, and stored scale/zero agree to float32 accuracy."""
    rng = np.random.default_rng(7)
    x = _bits(rng.standard_normal((3000, 128)) * rng.lognormal(0, 2.0, size=(3000, 1)))
    for bits in (2, 4):
        c0, s0, z0, t0 = O.rotate_quantize(x, 128, bits, 0)
        c1, s1, z1, t1 = O.rotate_quantize(x, 128, bits, 1)
        diff = c0 != c1
        assert diff.mean() < 1e-4
        assert np.all(np.abs(np.abs(t0[diff] - np.floor(t0[diff])) - 0.5) < 1e-4)
        m = np.maximum(np.abs(z0), np.abs(z0 + s0 * (2 ** bits - 1)))
        assert np.all(np.abs(s1 - s0) <= 1e-6 * np.maximum(s0, m / (2 ** bits - 1)))
        assert np.all(np.abs(z1 - z0) <= 1e-6 * m)


# ----------------------------------------------------------------------------- packing / placement

def pin_packing():
    for ex in _golden()["pack"]:
        got = O.pack_rows(np.array([ex["codes"]], dtype=np.uint8), ex["bits"])[0]
        assert list(got) == ex["bytes"], ex
    rng = np.random.default_rng(9)
    for bits in (2, 4):
        c = rng.integers(0, 2 ** bits, size=(50, 128)).astype(np.uint8)
        p = O.pack_rows(c, bits)
        assert p.shape == (50, 128 * bits // 8)
        assert np.array_equal(O.unpack_rows(p, bits), c)
        # bit-level spelled out: code i sits at bit (i * bits) of the little-endian row
        as_int = int.from_bytes(bytes(p[0]), "little")
        for i in range(128):
            assert (as_int >> (i * bits)) & (2 ** bits - 1) == c[0, i]


def _small_shape(bits=4, b=32, token_scale=0, hq=8, hkv=2, lens=(37, 16, 0, 70)):
    return W.config("tiny").with_(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, context_lens=tuple(lens),
                                  hadamard_block=b, bits=bits, token_scale=token_scale)


def _filled_cache(shape, plan):
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    slots = W.slots_for_positions(plan, shape.page_size, seq, pos)
    cache = O.PagedCache(plan.num_pages, shape.num_kv_heads, shape.page_size, shape.head_dim, shape.bits)
    diag = O.append(cache, k, v, slots, shape.hadamard_block, shape.token_scale)
    return cache, k, v, slots, diag


def pin_placement():
    """Gathering an appended cache back through its page table returns exactly the codes,
    scales and zeros of quantizing the same tokens contiguously; skipped slots and
    untouched slots keep their poison; the V tile interleaves 4 tokens per 32-bit word."""
    for bits, ts in ((4, 0), (2, 1)):
        shape = _small_shape(bits=bits, token_scale=ts)
        plan = W.plan_pages(shape)
        cache, k, v, slots, _ = _filled_cache(shape, plan)
        kc, ks, kz, _ = O.rotate_quantize(k.reshape(-1, 128), shape.hadamard_block, bits, ts)
        vc, vs, vz, _ = O.rotate_quantize(v.reshape(-1, 128), shape.hadamard_block, bits, ts)
        h_n = shape.num_kv_heads
        written = np.zeros((plan.num_pages, shape.page_size), dtype=bool)
        for i, slot in enumerate(slots):
            page, off = divmod(int(slot), shape.page_size)
            written[page, off] = True
            for h in range(h_n):
                r = i * h_n + h
                k_row, k_sz, v_row, v_sz = cache.read_token(page, off, h)
                assert np.array_equal(O.unpack_rows(k_row, bits), kc[r])
                assert np.array_equal(O.unpack_rows(v_row, bits), vc[r])
                assert k_sz[0] == ks[r] and k_sz[1] == kz[r] and v_sz[0] == vs[r] and v_sz[1] == vz[r]
                # raw byte addresses of the documented layout
                row = cache.row
                tile_k = cache.k_codes.reshape(plan.num_pages, h_n, -1)[page, h]
                tile_v = cache.v_codes.reshape(plan.num_pages, h_n, -1)[page, h]
                assert np.array_equal(tile_k[off * row:(off + 1) * row], k_row)
                idx = ((off // 4) * row + np.arange(row)) * 4 + off % 4
                assert np.array_equal(tile_v[idx], v_row)
        unwritten = ~written
        assert np.all(np.isnan(cache.k_sz.transpose(0, 2, 1, 3)[unwritten]))
        assert np.all(cache.k_codes.transpose(0, 2, 1, 3)[unwritten] == 0xAA)
    # a negative slot is skipped
    shape = _small_shape(lens=(8,))
    plan = W.plan_pages(shape)
    cache = O.PagedCache(plan.num_pages, 2, 16, 128, 4)
    k, v = W.draw_kv(shape, 8)
    O.append(cache, k, v, -np.ones(8, dtype=np.int64), 32, 0)
    assert np.all(cache.k_codes == 0xAA) and np.all(np.isnan(cache.v_sz))


# ----------------------------------------------------------------------------- attention

def _brute_softmax_attention(q, k, v, scale):
    """Python loops, float64: the textbook definition."""
    n = len(k)
    s = [scale * sum(float(q[d]) * float(k[j][d]) for d in range(len(q))) for j in range(n)]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    tot = sum(e)
    return [sum(e[j] / tot * float(v[j][d]) for j in range(n)) for d in range(len(v[0]))]


def pin_attention_definition():
    for ex in _golden()["attention"]:
        o = O.attend(np.array(ex["q"]), np.array(ex["k"]), np.array(ex["v"]), ex["scale"])
        assert np.allclose(o, ex["o"], rtol=1e-12, atol=1e-12), ex
    rng = np.random.default_rng(12)
    for n in (1, 3, 17):
        q = rng.standard_normal(8)
        k = rng.standard_normal((n, 8)) * 3
        v = rng.standard_normal((n, 8))
        got = O.attend(q, k, v, 0.5)
        assert np.allclose(got, _brute_softmax_attention(q, k, v, 0.5), rtol=1e-12, atol=1e-13)
    import torch
    q = torch.randn(1, 1, 1, 128, dtype=torch.float64, generator=torch.Generator().manual_seed(1))
    k = torch.randn(1, 1, 300, 128, dtype=torch.float64, generator=torch.Generator().manual_seed(2)) * 4
    v = torch.randn(1, 1, 300, 128, dtype=torch.float64, generator=torch.Generator().manual_seed(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0, 0].numpy()
    got = O.attend(q[0, 0, 0].numpy(), k[0, 0].numpy(), v[0, 0].numpy(), 1 / math.sqrt(128))
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)
    assert np.array_equal(O.attend(q[0, 0, 0].numpy(), np.zeros((0, 128)), np.zeros((0, 128)), 1.0), np.zeros(128))


def pin_attention_rotation_invariance():
    rng = np.random.default_rng(13)
    q = rng.standard_normal(128)
    k = rng.standard_normal((40, 128)) * 2
    v = rng.standard_normal((40, 128))
    base = O.attend(q, k, v, 0.1)
    for b in (2, 32, 128):
        r = O.rotation_matrix(128, b)
        rot = r.T @ O.attend(r @ q, k @ r.T, v @ r.T, 0.1)
        assert np.allclose(rot, base, rtol=1e-10, atol=1e-12)


def pin_decode_special_cases():
    """L = 1 returns the one dequantized V row un-rotated; equal keys give the mean of V;
    L = 0 gives zeros; query head h reads KV head h // g."""
    shape = _small_shape(hq=8, hkv=2, lens=(1, 20, 0, 33))
    plan = W.plan_pages(shape, extra_tokens=0)
    cache, k, v, slots, _ = _filled_cache(shape, plan)
    q = W.draw_q(shape)
    lens = np.array(shape.context_lens)
    out = O.decode(cache, q, plan.block_table, lens, shape.num_kv_heads, shape.hadamard_block)
    page0 = int(plan.block_table[0, 0])
    v_rows = O.dequant_page(cache, page0, shape.hadamard_block, 1, tensor="v")   # [H, ps, d]
    for h in range(8):
        assert np.allclose(out[0, h], v_rows[h // 4, 0], rtol=1e-6, atol=1e-6 * np.abs(v_rows).max())
    assert np.all(out[2] == 0)
    # equal keys: overwrite sequence 1's keys with one token's codes, then o = mean of V
    c2 = O.PagedCache(plan.num_pages, 2, 16, 128, 4)
    c2.k_codes[:], c2.v_codes[:], c2.k_sz[:], c2.v_sz[:] = cache.k_codes, cache.v_codes, cache.k_sz, cache.v_sz
    p_first = int(plan.block_table[1, 0])
    for j in range(20):
        page, off = int(plan.block_table[1, j // 16]), j % 16
        for h in range(2):
            c2.k_codes[page, h, off] = cache.k_codes[p_first, h, 0]
            c2.k_sz[page, h, off] = cache.k_sz[p_first, h, 0]
    out2 = O.decode(c2, q, plan.block_table, lens, 2, shape.hadamard_block)
    vs = [O.dequant_page(c2, int(plan.block_table[1, j // 16]), shape.hadamard_block, 1, tensor="v")[:, j % 16]
          for j in range(20)]
    mean_v = np.mean(np.stack(vs).astype(np.float64), axis=0)                  # [H, d]
    for h in range(8):
        assert np.allclose(out2[1, h], mean_v[h // 4], rtol=1e-5, atol=1e-5 * np.abs(mean_v).max())
    # GQA: constant V per KV head (value kvh + 1) survives rotate/quantize/unrotate
    shape3 = _small_shape(hq=8, hkv=2, lens=(24,))
    plan3 = W.identity_pages(shape3, extra_tokens=0)
    cache3 = O.PagedCache(plan3.num_pages, 2, 16, 128, 4)
    kk, _ = W.draw_kv(shape3, 24)
    vv = np.empty_like(kk)
    vv[:, 0, :] = _bits(np.ones(128))
    vv[:, 1, :] = _bits(np.full(128, 2.0))
    O.append(cache3, kk, vv, W.slots_for_positions(plan3, 16, *W.prefill_order(shape3)), 32, 0)
    out3 = O.decode(cache3, W.draw_q(shape3), plan3.block_table, np.array([24]), 2, 32)
    for h in range(8):
        assert np.allclose(out3[0, h], h // 4 + 1.0, rtol=2e-6), h


def pin_decode_page_table_invariance():
    """An identity page table and a shuffled one hold the same logical cache: identical outputs."""
    shape = _small_shape(hq=4, hkv=2, lens=(45, 3))
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    q = W.draw_q(shape)
    outs = []
    for plan in (W.identity_pages(shape, 0), W.plan_pages(shape, 0)):
        cache = O.PagedCache(plan.num_pages, 2, 16, 128, 4)
        O.append(cache, k, v, W.slots_for_positions(plan, 16, seq, pos), 32, 0)
        outs.append(O.decode(cache, q, plan.block_table, np.array(shape.context_lens), 2, 32))
    assert np.array_equal(outs[0], outs[1])


def pin_decode_vs_dense_unrotated():
    """Decode (rotated query against rotated cache, then R^T) equals plain attention of the
    un-rotated query against the un-rotated dequantized cache, written with dense matrices."""
    shape = _small_shape(hq=4, hkv=2, lens=(50,), b=64)
    plan = W.plan_pages(shape, 0)
    cache, k, v, slots, _ = _filled_cache(shape, plan)
    q = W.draw_q(shape)
    out = O.decode(cache, q, plan.block_table, np.array([50]), 2, 64, softmax_scale=0.07)
    for h in range(4):
        kv = h // 2
        kd = np.concatenate([O.dequant_page(cache, int(plan.block_table[0, p]), 64, 1, "k")[kv] for p in range(4)])[:50]
        vd = np.concatenate([O.dequant_page(cache, int(plan.block_table[0, p]), 64, 1, "v")[kv] for p in range(4)])[:50]
        qf = W.bf16_bits_to_f32(q[0, h]).astype(np.float64)
        s = 0.07 * kd.astype(np.float64) @ qf
        p = np.exp(s - s.max())
        o = (p / p.sum()) @ vd.astype(np.float64)
        assert np.allclose(out[0, h], o, rtol=1e-5, atol=1e-6 * np.abs(o).max()), h


def pin_decode_quantization_error_small():
    """Attention over the INT4 cache stays close to attention over the bf16 inputs (the
    method's premise: rotation + token-wise INT4 is nearly lossless); INT4 without rotation
    is worse on outlier channels."""
    shape = _small_shape(hq=8, hkv=2, lens=(256,), b=128)
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    q = W.draw_q(shape)
    kf, vf = W.bf16_bits_to_f32(k).astype(np.float64), W.bf16_bits_to_f32(v).astype(np.float64)
    errs = {}
    for b in (1, 128):
        plan = W.identity_pages(shape, 0)
        cache = O.PagedCache(plan.num_pages, 2, 16, 128, 4)
        O.append(cache, k, v, W.slots_for_positions(plan, 16, seq, pos), b, 0)
        out = O.decode(cache, q, plan.block_table, np.array([256]), 2, b)
        e = []
        for h in range(8):
            qf = W.bf16_bits_to_f32(q[0, h]).astype(np.float64)
            ref = O.attend(qf, kf[:, h // 4], vf[:, h // 4], 1 / math.sqrt(128))
            e.append(np.linalg.norm(out[0, h] - ref) / np.linalg.norm(ref))
        errs[b] = max(e)
    assert errs[128] < 0.2
    assert errs[128] < errs[1]


def pin_multi_query_attention():
    """Multi-query attention reduces to decode for one query per sequence, each later query
    sees exactly one more token (equal to decode over the shorter prefix), queries past q_lens are
    zero, and the result matches a dense causal softmax (torch SDPA with a causal mask) on the
    dequantized, rotated-back cache."""
    import torch
    shape = _small_shape(hq=4, hkv=2, lens=(40, 19, 7))
    plan = W.plan_pages(shape, 0)
    cache, k, v, slots, _ = _filled_cache(shape, plan)
    lens = np.array(shape.context_lens)
    rng = np.random.default_rng(31)
    qmax = 5
    q = _bits(rng.standard_normal((3, qmax, 4, 128)))
    q_lens = np.array([5, 1, 3])
    out = O.multi_query_attention(cache, q, q_lens, plan.block_table, lens, 2, 32)
    assert np.all(out[1, 1:] == 0) and np.all(out[2, 3:] == 0)
    # q_len 1 is the decode of that query
    dec = O.decode(cache, q[:, 0], plan.block_table, lens - q_lens + 1, 2, 32)
    for b in range(3):
        assert np.array_equal(out[b, 0], dec[b]), b
    # query j equals decode over the prefix ending at its own position
    for j in range(5):
        d_j = O.decode(cache, q[:, j], plan.block_table, lens - q_lens + j + 1, 2, 32)
        assert np.array_equal(out[0, j], d_j[0]), j
    # dense causal attention of the last 5 positions of sequence 0, with the rotation undone
    r = O.rotation_matrix(128, 32)
    for h in range(4):
        kh, vh = O.gather_sequence(cache, plan.block_table[0], 40, h // 2)
        qq = np.stack([r @ O.bf16_to_f32(q[0, j, h]).astype(np.float64) for j in range(5)])
        mask = np.arange(40)[None, :] <= (35 + np.arange(5))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qq)[None], torch.from_numpy(kh.astype(np.float64))[None],
            torch.from_numpy(vh.astype(np.float64))[None], attn_mask=torch.from_numpy(mask)[None])[0].numpy()
        ref = ref @ r                                   # R^T o, row vectors
        assert np.allclose(out[0, :, h], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max()), h


def pin_prerotated_query():
    """A query given already rotated (q_prerotated = 1) attends exactly like the plain query that
    rotates to it: decode(R q, 1) = decode(q, 0), and the same for multi-query attention. The
    rotated query y has small integer entries and q = R y is built with scipy's Hadamard matrix
    (b = 16: R = H_16 / 4), so both y and q are exact in bf16 and neither side of the check uses the
    oracle's own rotation."""
    import scipy.linalg
    b = 16
    shape = _small_shape(hq=4, hkv=2, b=b, lens=(40, 19, 7))
    plan = W.plan_pages(shape, 0)
    cache = _filled_cache(shape, plan)[0]
    lens = np.array(shape.context_lens)
    rng = np.random.default_rng(41)
    blk = scipy.linalg.hadamard(b).astype(np.float64) / 4.0
    r = np.kron(np.eye(128 // b), blk)
    y = rng.integers(-2, 3, size=(3, 2, 4, 128)).astype(np.float64)   # rotated queries
    q = y @ r.T                                                         # q = R y (R symmetric)
    assert np.array_equal(W.bf16_bits_to_f32(_bits(q)).astype(np.float64), q)   # exact in bf16
    y_bits, q_bits = _bits(y), _bits(q)
    plain = O.decode(cache, q_bits[:, 0], plan.block_table, lens, 2, b)
    pre = O.decode(cache, y_bits[:, 0], plan.block_table, lens, 2, b, q_prerotated=1)
    assert np.allclose(pre, plain, rtol=1e-6, atol=1e-6 * np.abs(plain).max())
    # the flag matters: the rotated query taken as a plain one is a different query
    assert not np.allclose(O.decode(cache, y_bits[:, 0], plan.block_table, lens, 2, b), plain, rtol=1e-3)
    q_lens = np.array([2, 1, 2])
    plain = O.multi_query_attention(cache, q_bits, q_lens, plan.block_table, lens, 2, b)
    pre = O.multi_query_attention(cache, y_bits, q_lens, plan.block_table, lens, 2, b, q_prerotated=1)
    assert np.allclose(pre, plain, rtol=1e-6, atol=1e-6 * np.abs(plain).max())


# ----------------------------------------------------------------------------- bf16 baseline

def pin_bf16_cache_layout():
    """Every token lands at the documented flat offsets: K at ((p*H + h)*ps + off)*d + c, V at
    (((p*H + h)*(ps/16) + off//16)*d + c)*16 + off%16; unwritten entries keep the poison; a
    negative slot is skipped."""
    ps, hkv, d, npages = 32, 2, 128, 3
    cache = O.PagedCacheBF16(npages, hkv, ps, d)
    rng = np.random.default_rng(21)
    slots = np.array([0, 5, 17, 31, 40, 95, -1], dtype=np.int64)
    k = rng.integers(0, 0x7F00, size=(len(slots), hkv, d)).astype(np.uint16)
    v = rng.integers(0, 0x7F00, size=(len(slots), hkv, d)).astype(np.uint16)
    O.append_bf16(cache, k, v, slots)
    kf, vf = cache.k.reshape(-1), cache.v.reshape(-1)
    written_k = np.zeros(kf.size, bool)
    written_v = np.zeros(vf.size, bool)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        p, off = divmod(int(slot), ps)
        for h in range(hkv):
            for c in range(d):
                ik = ((p * hkv + h) * ps + off) * d + c
                iv = (((p * hkv + h) * (ps // 16) + off // 16) * d + c) * 16 + off % 16
                assert kf[ik] == k[t, h, c] and vf[iv] == v[t, h, c]
                written_k[ik] = written_v[iv] = True
    assert np.all(kf[~written_k] == 0x7FC0) and np.all(vf[~written_v] == 0x7FC0)


def pin_decode_bf16_definition():
    """The bf16 baseline decode is softmax(q K^T / sqrt(d)) V over the gathered rows: equal to torch's
    scaled_dot_product_attention on the same (bf16-widened) tensors, to a brute-force loop on a
    tiny case, independent of the page table, zero for an empty sequence, and GQA maps query
    head h to KV head h // g."""
    import torch
    shape = _small_shape(hq=4, hkv=2, lens=(45, 3, 0))
    seq, pos = W.prefill_order(shape)
    k, v = W.draw_kv(shape, len(seq))
    q = W.draw_q(shape)
    lens = np.array(shape.context_lens)
    outs = []
    for plan in (W.identity_pages(shape, 0), W.plan_pages(shape, 0)):
        cache = O.PagedCacheBF16(plan.num_pages, 2, 16, 128)
        O.append_bf16(cache, k, v, W.slots_for_positions(plan, 16, seq, pos))
        outs.append(O.decode_bf16(cache, q, plan.block_table, lens, 2))
    assert np.array_equal(outs[0], outs[1])
    out = outs[0]
    assert np.all(out[2] == 0)
    kf = O.bf16_to_f32(k).astype(np.float64)
    vf = O.bf16_to_f32(v).astype(np.float64)
    start = 0
    for b, n in enumerate(shape.context_lens):
        if n == 0:
            continue
        for h in range(4):
            qq = torch.from_numpy(O.bf16_to_f32(q[b, h]).astype(np.float64))[None, None, None]
            kk = torch.from_numpy(kf[start:start + n, h // 2])[None, None]
            vv = torch.from_numpy(vf[start:start + n, h // 2])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, 0, 0].numpy()
            assert np.allclose(out[b, h], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max()), (b, h)
        start += n
    # brute force on the 3-token sequence, one head
    bf = _brute_softmax_attention(O.bf16_to_f32(q[1, 3]), kf[45:48, 1], vf[45:48, 1], 1 / math.sqrt(128))
    assert np.allclose(out[1, 3], bf, rtol=1e-5, atol=1e-7)


# ----------------------------------------------------------------------------- per-channel pages

def pin_pc_channel_quantizer():
    """Per-channel quantizer: the minimum and maximum are taken down each channel (a grid with
    per-channel gains and offsets is recovered exactly), a two-token page puts every channel's
    tokens on codes 0 and qmax, a constant channel gets scale 0, and the rounding error stays
    within half a step of its own channel."""
    rng = np.random.default_rng(21)
    for bits in (2, 4):
        qmax = 2 ** bits - 1
        c = rng.integers(0, qmax + 1, size=(64, 128))
        c[0], c[1] = 0, qmax                          # every channel reaches both ends
        gain = np.float32(2.0) ** rng.integers(-6, 4, size=128).astype(np.float32)
        off = rng.integers(-8, 8, size=128).astype(np.float32) / np.float32(4)
        u = (c * gain[None, :] + off[None, :]).astype(np.float32)
        codes, scale, zero, _ = O.quantize_channels(u, bits)
        assert np.array_equal(codes, c.astype(np.uint8))
        assert np.array_equal(scale, gain) and np.array_equal(zero, off)
        # two tokens: per channel the smaller one gets 0, the larger qmax
        two = rng.standard_normal((2, 128)).astype(np.float32)
        codes, scale, zero, _ = O.quantize_channels(two, bits)
        lo = two.argmin(axis=0)
        assert np.all(codes[lo, np.arange(128)] == 0) and np.all(codes[1 - lo, np.arange(128)] == qmax)
        assert np.array_equal(scale, (two.max(axis=0) - two.min(axis=0)) / np.float32(qmax))
        # constant channel
        u = rng.standard_normal((16, 128)).astype(np.float32)
        u[:, 5] = np.float32(-0.75)
        codes, scale, zero, _ = O.quantize_channels(u, bits)
        assert scale[5] == 0 and zero[5] == np.float32(-0.75) and np.all(codes[:, 5] == 0)
        # error bound of random data, per channel
        u = (rng.standard_normal((128, 128)) * rng.lognormal(0, 1, size=(1, 128))).astype(np.float32)
        codes, scale, zero, _ = O.quantize_channels(u, bits)
        deq = codes * scale[None, :].astype(np.float64) + zero[None, :]
        ulp = np.spacing(np.abs(u).max(axis=0, keepdims=True)).astype(np.float64)
        assert np.all(np.abs(deq - u) <= scale[None, :] / 2 + 4 * ulp)


def pin_pc_token_scale_equivariance():
    """Omni-token scaling makes the page's codes blind to each token's norm: multiplying one token
    by a power of two leaves every code and every channel (scale, zero) unchanged and multiplies
    that token's stored scale by the same factor (all steps exact). Without the scaling the
    small-norm tokens of a page with a wide norm spread would collapse onto one code; with it each
    token's relative error is bounded by the channel steps of unit-RMS tokens."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    xb = _bits(x)
    for bits in (2, 4):
        c0, s0, cp0, _ = O.quantize_page_pc(xb, 128, bits)
        for t, a in ((3, 4.0), (17, 0.125), (31, 1024.0)):
            x2 = x.copy()
            x2[t] *= np.float32(a)
            c1, s1, cp1, _ = O.quantize_page_pc(_bits(x2), 128, bits)
            assert np.array_equal(c1, c0) and np.array_equal(cp1, cp0)
            want = s0.copy()
            want[t] *= np.float32(a)
            assert np.array_equal(s1, want)
        # norm spread of 1e6 across the page: every token keeps a bounded relative error
        wide = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-7, 7, size=(64, 1)))).astype(np.float32)
        wb = _bits(wide)
        codes, s, cp, _ = O.quantize_page_pc(wb, 128, bits)
        y = O.rotate_f32(O.bf16_to_f32(wb), 128).astype(np.float64)
        deq = (codes * cp[0].astype(np.float64) + cp[1]) * s[:, None].astype(np.float64)
        rel = np.linalg.norm(deq - y, axis=1) / np.linalg.norm(y, axis=1)
        bound = np.sqrt(np.mean(cp[0].astype(np.float64) ** 2)) / 2 * 1.0001
        assert np.all(rel <= bound), (bits, rel.max(), bound)


def pin_pc_layout_matches_token_cache():
    """The per-channel cache stores codes exactly where the token-wise cache does (so the two read
    paths share their code loads), token scales per token and (scale, zero) per channel."""
    rng = np.random.default_rng(23)
    for bits in (2, 4):
        ps = 32
        pc = O.PagedCachePC(3, 2, ps, 128, bits)
        tw = O.PagedCache(3, 2, ps, 128, bits)
        kc = rng.integers(0, 2 ** bits, size=(ps, 128)).astype(np.uint8)
        vc = rng.integers(0, 2 ** bits, size=(ps, 128)).astype(np.uint8)
        ks, vs = rng.random(ps).astype(np.float32), rng.random(ps).astype(np.float32)
        kcp, vcp = rng.random((2, 128)).astype(np.float32), rng.random((2, 128)).astype(np.float32)
        pc.write_page(2, 1, kc, ks, kcp, vc, vs, vcp)
        kp, vp = O.pack_rows(kc, bits), O.pack_rows(vc, bits)
        for t in range(ps):
            tw.write_token(2, t, 1, kp[t], 0.0, 0.0, vp[t], 0.0, 0.0)
        assert np.array_equal(pc.k_codes, tw.k_codes) and np.array_equal(pc.v_codes, tw.v_codes)
        for tensor, c, s, cp in (("k", kc, ks, kcp), ("v", vc, vs, vcp)):
            rc, rs, rcp = pc.read_page(2, 1, tensor)
            assert np.array_equal(rc, c) and np.array_equal(rs, s) and np.array_equal(rcp, cp)
        assert np.all(np.isnan(pc.k_s[:2])) and np.all(np.isnan(pc.v_cp[2, 0]))


def _pc_case(lens, ps, bits, hb, rng, exact):
    """A per-channel cache holding the complete pages of sequences of the given lengths, their
    tails, and the raw K/V of every token. exact: tokens +-a_t with a_t a power of two and both
    signs in every channel of every page, so that (with hb = 1) each page is quantized exactly."""
    h_n, d = 2, 128
    n_pages_seq = [n // ps for n in lens]
    bt = np.full((len(lens), max(1, max(n_pages_seq))), -1, dtype=np.int32)
    order = rng.permutation(sum(n_pages_seq) + 2)
    raw_k, raw_v = [], []
    pages_k, pages_v, ids = [], [], []
    tail_k = np.zeros((len(lens), ps, h_n, d), dtype=np.uint16)
    tail_v = np.zeros((len(lens), ps, h_n, d), dtype=np.uint16)
    nxt = 0
    for b, n in enumerate(lens):
        if exact:
            sign = np.where(rng.random((n, h_n, d)) < 0.5, -1.0, 1.0)
            for j in range(n // ps):
                sign[j * ps, :, :], sign[j * ps + 1, :, :] = -1.0, 1.0
            amp = np.float32(2.0) ** rng.integers(-3, 4, size=(n, h_n, 1))
            k = (sign * amp).astype(np.float32)
            v = (np.roll(sign, 1, axis=0) * amp[::-1]).astype(np.float32)
        else:
            k = (rng.standard_normal((n, h_n, d)) * rng.lognormal(0, 1, size=(n, h_n, 1))).astype(np.float32)
            v = rng.standard_normal((n, h_n, d)).astype(np.float32)
        kb, vb = _bits(k), _bits(v)
        raw_k.append(O.bf16_to_f32(kb))
        raw_v.append(O.bf16_to_f32(vb))
        for j in range(n // ps):
            bt[b, j] = order[nxt]
            ids.append(order[nxt])
            nxt += 1
            pages_k.append(kb[j * ps:(j + 1) * ps])
            pages_v.append(vb[j * ps:(j + 1) * ps])
        full = (n // ps) * ps
        tail_k[b, :n - full] = kb[full:]
        tail_v[b, :n - full] = vb[full:]
    cache = O.PagedCachePC(len(order), h_n, ps, d, bits)
    if ids:
        O.write_pages_pc(cache, np.concatenate(pages_k), np.concatenate(pages_v), np.array(ids), hb)
    return cache, bt, tail_k, tail_v, raw_k, raw_v


def pin_pc_decode_definition():
    """Decode over per-channel pages plus the residual window is softmax attention over every
    token of the sequence: exact (up to the float32 rounding of the step) when each page's
    tokens sit on its quantization grid, for
    sequences with only a tail, only complete pages, both, and none; close to the dense attention
    (within the quantization error) for random data with the rotation."""
    import torch
    rng = np.random.default_rng(24)
    ps = 32
    lens = [0, 7, 64, 77, 32]
    for bits in (2, 4):
        cache, bt, tk, tv, rk, rv = _pc_case(lens, ps, bits, 1, rng, exact=True)
        q = _bits(rng.standard_normal((len(lens), 4, 128)))
        out = O.decode_pc(cache, q, bt, np.array(lens), tk, tv, 2, 1)
        assert np.all(out[0] == 0)
        for b, n in enumerate(lens):
            if n == 0:
                continue
            for h in range(4):
                qq = torch.from_numpy(O.bf16_to_f32(q[b, h]).astype(np.float64))[None, None, None]
                kk = torch.from_numpy(rk[b][:, h // 2].astype(np.float64))[None, None]
                vv = torch.from_numpy(rv[b][:, h // 2].astype(np.float64))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, 0, 0].numpy()
                # the step 2 / qmax is not exact in float32: about 3e-8 relative per key
                assert np.allclose(out[b, h], ref, rtol=2e-5, atol=2e-5 * np.abs(ref).max()), (bits, b, h)
    # random data, real rotation: the same as attention over keys and values rebuilt by hand from
    # the cache arrays (codes unpacked with shifts, scipy's Hadamard matrix for the rotation)
    import scipy.linalg
    lens = [96, 45]
    cache, bt, tk, tv, rk, rv = _pc_case(lens, ps, 4, 128, rng, exact=False)
    q = _bits(rng.standard_normal((2, 4, 128)))
    out = O.decode_pc(cache, q, bt, np.array(lens), tk, tv, 2, 128)
    rot = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128)
    for b, n in enumerate(lens):
        for kvh in range(2):
            ks, vs = [], []
            for j in range(n // ps):
                pg = bt[b, j]
                kbyte = cache.k_codes[pg, kvh].astype(np.int64)                      # [ps, 64]
                kcode = np.stack([kbyte & 15, kbyte >> 4], axis=-1).reshape(ps, 128)
                vbyte = cache.v_codes[pg, kvh].transpose(0, 2, 1).reshape(ps, 64).astype(np.int64)
                vcode = np.stack([vbyte & 15, vbyte >> 4], axis=-1).reshape(ps, 128)
                for code, sc, cp, acc in ((kcode, cache.k_s, cache.k_cp, ks), (vcode, cache.v_s, cache.v_cp, vs)):
                    u = code * cp[pg, kvh, 0].astype(np.float64) + cp[pg, kvh, 1].astype(np.float64)
                    acc.append((u * sc[pg, kvh][:, None].astype(np.float64)) @ rot)
            full = (n // ps) * ps
            ks.append(O.bf16_to_f32(tk[b, :n - full, kvh]).astype(np.float64))
            vs.append(O.bf16_to_f32(tv[b, :n - full, kvh]).astype(np.float64))
            kk = torch.from_numpy(np.concatenate(ks))[None, None]
            vv = torch.from_numpy(np.concatenate(vs))[None, None]
            for h in (2 * kvh, 2 * kvh + 1):
                qq = torch.from_numpy(O.bf16_to_f32(q[b, h]).astype(np.float64))[None, None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, 0, 0].numpy()
                assert np.allclose(out[b, h], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max()), (b, h)

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

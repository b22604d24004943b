"""CPU checks of the test-side helpers: the vectorised host-cache builder writes exactly what
the oracle's per-token append writes, and the layout views read the documented bytes."""
import numpy as np

import parity_helpers as H
from oracle import kvq_oracle as O
from paged_decode_attention_amd import workloads as W


def test_host_cache_builder_matches_oracle_append():
    for bits, ts, hb in ((4, 0, 32), (2, 1, 128), (4, 0, 1)):
        s = W.config("tiny").with_(batch=3, num_q_heads=4, num_kv_heads=2, context_lens=(40, 17, 5), bits=bits,
                                   token_scale=ts, hadamard_block=hb)
        plan = W.plan_pages(s)
        seq, pos = W.prefill_order(s)
        k, v = W.draw_kv(s, len(seq))
        slots = W.slots_for_positions(plan, 16, seq, pos)
        slots[3] = -1
        ref = O.PagedCache(plan.num_pages, 2, 16, 128, bits)
        O.append(ref, k, v, slots, hb, ts)
        got, _ = H.host_cache_from_oracle(k, v, slots, plan.num_pages, 16, hb, bits, ts)
        assert np.array_equal(got.k_codes, ref.k_codes) and np.array_equal(got.v_codes, ref.v_codes)
        assert np.array_equal(got.k_sz, ref.k_sz, equal_nan=True)
        assert np.array_equal(got.v_sz, ref.v_sz, equal_nan=True)
        kc, vc = H.cache_codes(ref)
        for i in (0, 7, 40):
            page, off = divmod(int(slots[i]), 16)
            k_row, _, v_row, _ = ref.read_token(page, off, 1)
            assert np.array_equal(kc[page, 1, off], O.unpack_rows(k_row, bits))
            assert np.array_equal(vc[page, 1, off], O.unpack_rows(v_row, bits))


def test_agreement_rules_reject_planted_errors():
    rng = np.random.default_rng(0)
    ref = rng.integers(0, 16, size=(4, 128)).astype(np.uint8)
    t = ref.astype(np.float64) + rng.uniform(-0.4, 0.4, size=ref.shape)
    H.check_codes(ref.copy(), ref, t, "same")
    bad = ref.copy()
    bad[0, 0] ^= 1
    try:
        H.check_codes(bad, ref, t, "planted")
        raise AssertionError("planted code error not detected")
    except AssertionError as e:
        assert "planted" in str(e)
    o = rng.standard_normal((3, 128))
    H.check_attention(o + 1e-6, o, "close")
    try:
        H.check_attention(o * 1.01, o, "far")
        raise AssertionError("planted attention error not detected")
    except AssertionError as e:
        assert "far" in str(e)

"""The seeded input generators: deterministic, the shapes and distributions stated for
each workload, and page plans that never hand out a page twice."""
import numpy as np

from paged_decode_attention_amd import workloads as W


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, np.inf], dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0                  # tie -> even (down)
    assert back[2] == np.float32(1.0 + 4 * 2 ** -8)           # tie -> even (up)
    assert back[3] == -2.5 and np.isinf(back[5])


def test_deterministic_and_distribution():
    s = W.config("tiny")
    k1, v1 = W.draw_kv(s, 512)
    k2, v2 = W.draw_kv(s, 512)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert k1.shape == (512, 8, 128) and k1.dtype == np.uint16
    kf = W.bf16_bits_to_f32(k1).astype(np.float64)
    ch = W.outlier_channels(s)
    assert len(ch) == 4
    norms = np.linalg.norm(kf, axis=-1)                        # [T, H]
    # per-token factor is shared across heads: head norms of a token move together
    assert np.corrcoef(np.log(norms[:, 0]), np.log(norms[:, 1]))[0, 1] > 0.8
    # outlier channels carry ~10x the magnitude of the rest
    rms = np.sqrt((kf ** 2).mean(axis=(0, 1)))
    others = np.delete(rms, ch)
    assert rms[ch].min() > 5 * others.max()
    assert not np.array_equal(k1, v1)
    q = W.draw_q(s)
    assert q.shape == (1, 8, 128)


def test_page_plans():
    for name in ("tiny", "llama3_8b", "sweep_b32", "oscar_int2"):
        s = W.config(name)
        plan = W.plan_pages(s)
        used = plan.block_table[plan.block_table >= 0]
        assert len(np.unique(used)) == len(used)
        assert used.max() < plan.num_pages
        need = (np.asarray(s.context_lens) + 1 + 15) // 16
        assert np.array_equal((plan.block_table >= 0).sum(axis=1), need)
        seq, pos = W.prefill_order(s)
        slots = W.slots_for_positions(plan, 16, seq, pos)
        assert len(np.unique(slots)) == len(slots)


def test_sweep_lengths_and_chunks():
    s = W.config("sweep_b256")
    lens = np.asarray(s.context_lens)
    assert lens.min() >= 512 and lens.max() <= 8192 and len(lens) == 256
    c = W.config("oscar_int2", batch=3, context_lens=(1100, 600, 40))
    calls = W.chunk_schedule(c)
    seen = {b: [] for b in range(3)}
    for seq, pos in calls:
        for b, p in zip(seq, pos):
            seen[int(b)].append(int(p))
    for b, n in enumerate(c.context_lens):
        assert seen[b] == list(range(n))
    first = calls[0]
    assert all(1 <= (first[0] == b).sum() <= 15 for b in range(3))

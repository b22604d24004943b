"""Plant plausible mistakes in the CPU oracle (on the CPU, in this process only) and check
that at least one pin catches each: the pins are sensitive to a dropped term, a wrong sign
or index, a transposed operand, a wrong rounding rule or a misplaced byte."""
import math

import numpy as np
import pytest

import oracle_pins as P
from oracle import kvq_oracle as O


def _caught(monkeypatch_fn):
    """Run every pin with the planted mistake applied; True if one of them fails."""
    mp = pytest.MonkeyPatch()
    try:
        monkeypatch_fn(mp)
        for pin in P.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                return pin.__name__
        return None
    finally:
        mp.undo()


_real_hadamard = O.hadamard
_real_quantize = O.quantize_rows
_real_pack = O.pack_rows
_real_attend = O.attend
_real_rotate = O.rotate_f32


def m_hadamard_sign(mp):
    def bad(n):
        h = _real_hadamard(n).copy()
        if n >= 4:
            h[1, 2] = -h[1, 2]
        return h
    mp.setattr(O, "hadamard", bad)


def m_hadamard_row_order(mp):
    def bad(n):
        h = _real_hadamard(n)
        return h[::-1].copy()          # rows reversed: still orthogonal, wrong order
    mp.setattr(O, "hadamard", bad)


def m_rotation_norm(mp):
    # 1/sqrt(b) applied twice
    mp.setattr(O, "rotate_f32", lambda x, b: _real_rotate(x, b) * np.float32(1.0 / math.sqrt(b)))


def m_round_half_up(mp):
    def bad(u, bits):
        c, s, z, t = _real_quantize(u, bits)
        u = np.asarray(u, dtype=np.float32)
        safe = np.where(s != 0, s, np.float32(1))
        tf = (u - z[:, None]) / safe[:, None]
        c2 = np.clip(np.floor(tf + np.float32(0.5)), 0, 2 ** bits - 1).astype(np.uint8)
        c2[s == 0] = 0
        return c2, s, z, t
    mp.setattr(O, "quantize_rows", bad)


def m_qmax_off_by_one(mp):
    def bad(u, bits):
        u = np.asarray(u, dtype=np.float32)
        mn, mx = u.min(axis=-1), u.max(axis=-1)
        s = (mx - mn) / np.float32(2 ** bits)
        safe = np.where(s != 0, s, np.float32(1))
        c = np.clip(np.rint((u - mn[:, None]) / safe[:, None]), 0, 2 ** bits - 1).astype(np.uint8)
        return c, s, mn, np.zeros(u.shape)
    mp.setattr(O, "quantize_rows", bad)


def m_zero_is_max(mp):
    def bad(u, bits):
        c, s, z, t = _real_quantize(u, bits)
        return c, s, np.asarray(u, dtype=np.float32).max(axis=-1), t
    mp.setattr(O, "quantize_rows", bad)


def m_pack_high_first(mp):
    def bad(codes, bits):
        per = 8 // bits
        c = np.asarray(codes, dtype=np.uint8)
        c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per)).astype(np.uint32)
        out = np.zeros(c.shape[:-1], dtype=np.uint32)
        for k in range(per):
            out |= c[..., k] << (bits * (per - 1 - k))
        return out.astype(np.uint8)
    mp.setattr(O, "pack_rows", bad)


def m_v_interleave_swapped(mp):
    def write_token(self, page, off, head, k_row, k_scale, k_zero, v_row, v_scale, v_zero):
        self.k_codes[page, head, off, :] = k_row
        self.v_codes[page, head, off % 4, :, off // 4 % 4] = v_row
        self.k_sz[page, head, off] = (k_scale, k_zero)
        self.v_sz[page, head, off] = (v_scale, v_zero)

    def read_token(self, page, off, head):
        return (self.k_codes[page, head, off, :], self.k_sz[page, head, off],
                self.v_codes[page, head, off % 4, :, off // 4 % 4], self.v_sz[page, head, off])
    mp.setattr(O.PagedCache, "write_token", write_token)
    mp.setattr(O.PagedCache, "read_token", read_token)


def m_no_softmax_scale(mp):
    mp.setattr(O, "attend", lambda q, k, v, s: _real_attend(q, k, v, 1.0))


def m_no_inverse_rotation(mp):
    real_rm = O.rotation_matrix

    def decode(cache, q_bits, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale=0.0,
               q_prerotated=0, heads=None):
        bsz, hq, d = q_bits.shape
        g = hq // num_kv_heads
        scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(d)
        r = real_rm(d, hadamard_block)
        out = np.zeros((bsz, hq, d), dtype=np.float32)
        for b in range(bsz):
            for h in range(hq):
                kh, vh = O.gather_sequence(cache, block_table[b], int(context_lens[b]), h // g)
                q = O.bf16_to_f32(q_bits[b, h]).astype(np.float64)
                out[b, h] = O.attend(r @ q, kh, vh, scale)          # R^T forgotten
        return out
    mp.setattr(O, "decode", decode)


def m_gqa_modulo(mp):
    real_decode = O.decode

    def decode(cache, q_bits, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale=0.0,
               q_prerotated=0, heads=None):
        bsz, hq, d = q_bits.shape
        g = hq // num_kv_heads
        # query head h mapped to KV head h % num_kv_heads instead of h // g
        perm = np.array([(h % num_kv_heads) * g + (h // num_kv_heads) for h in range(hq)]) if g > 1 else np.arange(hq)
        out = real_decode(cache, q_bits[:, perm], block_table, context_lens, num_kv_heads, hadamard_block,
                          softmax_scale, q_prerotated)
        inv = np.argsort(perm)
        return out[:, inv]
    mp.setattr(O, "decode", decode)


def m_gather_wrong_offset(mp):
    real = O.gather_sequence

    def bad(cache, block_table_row, length, head):
        kh, vh = real(cache, block_table_row, length, head)
        return kh[::-1].copy(), vh                                    # keys paired with the wrong values
    mp.setattr(O, "gather_sequence", bad)


def m_rms_no_sqrt(mp):
    real = O.token_rms
    mp.setattr(O, "token_rms", lambda y: real(y) ** 2)             # mean square, not its root


def m_rms_max_abs(mp):
    def bad(y):
        s = np.abs(np.asarray(y, dtype=np.float32)).max(axis=-1)   # a max-abs norm instead of the RMS
        s[s == 0] = np.float32(1.0)
        return s
    mp.setattr(O, "token_rms", bad)


def m_bf16_v_token_major(mp):
    def write_token(self, page, off, head, k_row, v_row):
        self.k[page, head, off, :] = k_row
        self.v.reshape(self.num_pages, self.kv_heads, self.page_size, self.head_dim)[page, head, off, :] = v_row

    def read_token(self, page, off, head):
        return (self.k[page, head, off, :],
                self.v.reshape(self.num_pages, self.kv_heads, self.page_size, self.head_dim)[page, head, off, :])
    mp.setattr(O.PagedCacheBF16, "write_token", write_token)
    mp.setattr(O.PagedCacheBF16, "read_token", read_token)


def m_bf16_gqa_modulo(mp):
    real = O.decode_bf16

    def bad(cache, q_bits, block_table, context_lens, num_kv_heads, softmax_scale=0.0, heads=None):
        hq = q_bits.shape[1]
        g = hq // num_kv_heads
        perm = np.array([(h % num_kv_heads) * g + (h // num_kv_heads) for h in range(hq)]) if g > 1 else np.arange(hq)
        out = real(cache, q_bits[:, perm], block_table, context_lens, num_kv_heads, softmax_scale)
        return out[:, np.argsort(perm)]
    mp.setattr(O, "decode_bf16", bad)


def m_mq_off_by_one(mp):
    real = O.multi_query_attention

    def bad(cache, q_bits, q_lens, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale=0.0,
            q_prerotated=0, rows=None):
        # each query also sees the token after its own position
        return real(cache, q_bits, q_lens, block_table, np.asarray(context_lens) + 1, num_kv_heads, hadamard_block,
                    softmax_scale, q_prerotated, rows)
    mp.setattr(O, "multi_query_attention", bad)


def m_pc_token_axis(mp):
    # the page quantized token by token (the token-wise quantizer) instead of channel by channel
    mp.setattr(O, "quantize_channels", lambda u, bits: _real_quantize(u, bits))


def m_pc_no_token_scale(mp):
    real = O.quantize_page_pc

    def bad(x_bits, b, bits):
        y = O.rotate_f32(O.bf16_to_f32(x_bits), b)
        codes, sc, zr, t = O.quantize_channels(y, bits)              # the scaling step left out
        return codes, np.ones(len(y), np.float32), np.stack([sc, zr]).astype(np.float32), t
    mp.setattr(O, "quantize_page_pc", bad)


def m_pc_dequant_without_s(mp):
    def bad(cache, page, head, tensor):
        codes, s, cp = cache.read_page(page, head, tensor)
        return codes.astype(np.float64) * cp[0].astype(np.float64)[None, :] + cp[1].astype(np.float64)[None, :]
    mp.setattr(O, "dequant_page_pc", bad)


def m_pc_tail_off_by_one(mp):
    real = O.decode_pc

    def bad(cache, q_bits, block_table, context_lens, tail_k_bits, tail_v_bits, num_kv_heads, hadamard_block,
            softmax_scale=0.0, heads=None):
        return real(cache, q_bits, block_table, context_lens, np.roll(tail_k_bits, 1, axis=1), tail_v_bits,
                    num_kv_heads, hadamard_block, softmax_scale, heads)
    mp.setattr(O, "decode_pc", bad)


def m_pc_v_token_major(mp):
    def write_page(self, page, head, kc, ks, kcp, vc, vs, vcp):
        self.k_codes[page, head] = O.pack_rows(kc, self.bits)
        self.v_codes[page, head] = O.pack_rows(vc, self.bits).reshape(self.page_size // 4, 4, self.row).transpose(0, 1, 2).reshape(self.page_size // 4, self.row, 4)
        self.k_s[page, head], self.v_s[page, head] = ks, vs
        self.k_cp[page, head], self.v_cp[page, head] = kcp, vcp
    mp.setattr(O.PagedCachePC, "write_page", write_page)


def m_prerotated_rotated_again(mp):
    # the pre-rotated query is rotated once more (the flag ignored) in decode and multi-query attention
    real_dec, real_mq = O.decode, O.multi_query_attention

    def dec(cache, q_bits, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale=0.0,
            q_prerotated=0, heads=None):
        return real_dec(cache, q_bits, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale, 0,
                        heads)

    def mq(cache, q_bits, q_lens, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale=0.0,
           q_prerotated=0, rows=None):
        return real_mq(cache, q_bits, q_lens, block_table, context_lens, num_kv_heads, hadamard_block, softmax_scale,
                       0, rows)
    mp.setattr(O, "decode", dec)
    mp.setattr(O, "multi_query_attention", mq)


MUTATIONS = [m_hadamard_sign, m_hadamard_row_order, m_rotation_norm, m_round_half_up, m_qmax_off_by_one,
             m_zero_is_max, m_pack_high_first, m_v_interleave_swapped, m_no_softmax_scale,
             m_no_inverse_rotation, m_gqa_modulo, m_gather_wrong_offset, m_rms_no_sqrt, m_rms_max_abs, m_bf16_v_token_major, m_bf16_gqa_modulo, m_mq_off_by_one,
             m_pc_token_axis, m_pc_no_token_scale, m_pc_dequant_without_s, m_pc_tail_off_by_one, m_pc_v_token_major,
             m_prerotated_rotated_again]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mutation):
    caught_by = _caught(mutation)
    assert caught_by is not None, f"no pin catches {mutation.__name__}"

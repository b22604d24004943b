"""CPU oracle for the rotated low-bit paged KV cache (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call this module. The product path (the HIP library and its Python
binding) never does, and shares no code with it.

It is the plain definition of what the method computes, written out slowly with numpy:

* Write path -- from the SAW-INT4 abstract ("SAW-INT4: System-Aware 4-Bit KV-Cache
  Quantization for Real-World LLM Serving", fugumt.com paper page, Abstract): every new
  K/V head vector is rotated by a block-diagonal Hadamard matrix and then quantized
  token-wise to INT4, inside a paged cache layout. From the OScaR summary ("OScaR:
  Occam's Razor for Extreme KV Cache Quantization in LLMs", zhichai.net, section "The
  OScaR Framework", the formula V-hat = Quant(S (R V))): rotate, then scale each token,
  then quantize; used at INT2.
* Read path -- decode attention over the dequantized pages (the fused dequantize-and-
  attend kernel of the ainews.cool "Technical Deep Dive"; the paged INT2 attention kernel
  of the OSCAR abstract on the thelatestinai.com page): the query is rotated by the same
  matrix, scores are softmax(q k / sqrt(D)), and one inverse rotation on the output undoes
  the rotation of V.

* Several queries per sequence (chunked prefill, speculative verification) -- the same attention
  with a causal limit per query: the paged low-bit attention of the OSCAR abstract applied to the
  prefill side.
* Per-channel pages (``PagedCachePC``, ``write_pages_pc``, ``decode_pc``) -- the per-channel
  reading of OScaR (OScaR abstract on the openalex page: the method moves per-channel quantization forward;
  zhichai.net summary, "Root Cause: Token Norm Imbalance" and "The OScaR Framework"): per-token
  scaling after the rotation, then one (scale, zero) per channel shared by the tokens of a page;
  a sequence's unfinished last page stays in bf16 until it is complete.
* Baseline -- attention over an unquantized bf16 paged cache (``PagedCacheBF16``,
  ``append_bf16``, ``decode_bf16``): the BF16 split decode the OScaR abstract (thelatestinai.com
  page) measures its speed-up against, used to put the low-bit path's speed next to it.

Precision: the rotation's +-1 sums are formed exactly (float64, which holds every sum of
at most 128 bf16 values here) and rounded once to float32, then multiplied by the float32
constant 1/sqrt(b); the quantizer runs in float32 with IEEE division and round-half-to-
even; the optional per-token scale is the float32 rounding of an RMS computed in float64;
attention accumulates in float64 and returns float32.

Readings of points the pages leave open:
  * Hadamard: Sylvester order, H[i, j] = (-1)^popcount(i & j), normalised by 1/sqrt(b), no
    random signs; blocks are contiguous channel ranges; the same matrix for K, V and Q.
  * Quantizer: scale = (max - min) / (2^bits - 1), zero = min (a float offset),
    code = clamp(rint((u - min) / scale), 0, 2^bits - 1); dequant = code * scale + zero.
    A constant vector gets scale 0, zero = min and all-zero codes.
  * Per-token scaling (OScaR): s = RMS of the rotated vector (s = 1 when it is 0),
    u = y / s; the stored scale and zero are scale_u * s and min_u * s.
    Parity unpinned: the pages name no norm for s, so RMS is a reading that nothing on
    the pages can confirm. ``token_rms`` itself is pinned to closed forms. The choice
    barely matters here: any positive s cancels in the codes, and the stored scale and
    zero change only by float32 rounding.
  * Packing: low bits first (INT4: channel 2j in the low nibble of byte j).
  * Layout (caller-owned arrays, all row-major):
      K codes  [num_pages][kv_heads][page_size][row]               row = D * bits / 8 bytes
      V codes  [num_pages][kv_heads][page_size / 4][row][4]        byte (t, j) at
               ((t // 4) * row + j) * 4 + t % 4 inside a page-head tile
      K/V sz   [num_pages][kv_heads][page_size][2] float32 = {scale, zero}
    slot = page * page_size + offset; a negative slot skips the token.
  * GQA: query head h reads KV head h // (num_q_heads // num_kv_heads).
  * Per-channel pages: the page is the group that shares one (scale, zero) per channel; the
    per-token scale is the same RMS (parity unpinned as to the norm); a page is quantized
    once complete, and a sequence's newest (length mod page_size) tokens are attended in bf16.
  * Softmax scale 1/sqrt(D) unless given; output float32, in the original (un-rotated)
    basis; a sequence of length 0 yields zeros.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "hadamard", "rotation_matrix", "rotate_f32", "token_rms", "quantize_rows",
    "rotate_quantize", "pack_rows", "unpack_rows", "PagedCache", "append",
    "gather_sequence", "attend", "decode", "dequant_page", "bf16_to_f32",
    "PagedCacheBF16", "append_bf16", "decode_bf16", "multi_query_attention",
    "quantize_channels", "PagedCachePC", "quantize_page_pc", "quantize_rotated_page_pc", "write_pages_pc",
    "dequant_page_pc", "decode_pc",
]


# ----------------------------------------------------------------------------- inputs

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (bf16 is the top half of a float32, so this is exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- rotation

def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two): H[i, j] = (-1)^popcount(i & j).

    This is the +-1 matrix of the block-diagonal Hadamard rotation in the SAW-INT4 abstract;
    unnormalised, so H H^T = n I.
    """
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.empty((n, n), dtype=np.int64)
    for i in range(n):
        for j in range(n):
            h[i, j] = -1 if bin(i & j).count("1") % 2 else 1
    return h


def rotation_matrix(d: int, b: int) -> np.ndarray:
    """R = blockdiag(H_b, ..., H_b) / sqrt(b), float64 [d, d] (orthonormal, symmetric)."""
    if d % b:
        raise ValueError("Hadamard block must divide head_dim")
    r = np.zeros((d, d), dtype=np.float64)
    hb = hadamard(b).astype(np.float64) / math.sqrt(b)
    for s in range(0, d, b):
        r[s:s + b, s:s + b] = hb
    return r


def rotate_f32(x: np.ndarray, b: int) -> np.ndarray:
    """y = R x for each row of x (float32 [N, d]), as a dense matmul.

    The +-1 sums are formed exactly and rounded once to float32; the float32 constant
    1/sqrt(b) is then applied in float32.
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    hblk = np.zeros((d, d), dtype=np.float64)
    hb = hadamard(b).astype(np.float64)
    for s in range(0, d, b):
        hblk[s:s + b, s:s + b] = hb
    sums = (x.astype(np.float64) @ hblk.T).astype(np.float32)
    return sums * np.float32(1.0 / math.sqrt(b))


# ----------------------------------------------------------------------------- quantizer

def token_rms(y: np.ndarray) -> np.ndarray:
    """Per-token scale of the OScaR scaling step: float32(sqrt(mean(y^2))), 1 where that is 0."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    s = np.sqrt(np.mean(y64 * y64, axis=-1)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    return s


def quantize_rows(u: np.ndarray, bits: int):
    """Token-wise asymmetric quantization of float32 rows u [N, d].

    Returns (codes uint8 [N, d], scale float32 [N], zero float32 [N], t float64 [N, d]),
    where t is the pre-rounding value (u - min) / scale recomputed in float64 from the
    float32 operands (used only to find elements sitting on a rounding boundary).
    """
    u = np.asarray(u, dtype=np.float32)
    qmax = np.float32(2 ** bits - 1)
    mn = u.min(axis=-1)
    mx = u.max(axis=-1)
    scale = (mx - mn) / qmax                            # float32 subtract, IEEE divide
    live = scale != 0
    safe = np.where(live, scale, np.float32(1.0))
    tf = (u - mn[:, None]) / safe[:, None]              # float32, IEEE divide
    codes = np.clip(np.rint(tf), 0, qmax).astype(np.uint8)
    codes[~live] = 0
    t = (u.astype(np.float64) - mn[:, None].astype(np.float64)) / safe[:, None].astype(np.float64)
    t[~live] = 0.0
    return codes, scale.astype(np.float32), mn.astype(np.float32), t


def rotate_quantize(x_bits: np.ndarray, b: int, bits: int, token_scale: int):
    """The write-path value transform for rows of bf16 bits [N, d].

    Returns (codes, stored_scale, stored_zero, t) with the meaning of ``quantize_rows``.
    """
    x = bf16_to_f32(x_bits)
    y = rotate_f32(x, b)
    if token_scale:
        s = token_rms(y)
        u = y / s[:, None]                              # float32, IEEE divide
        codes, sc, zr, t = quantize_rows(u, bits)
        return codes, (sc * s).astype(np.float32), (zr * s).astype(np.float32), t
    return quantize_rows(y, bits)


# ----------------------------------------------------------------------------- packing

def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [..., d] (values < 2^bits) into bytes [..., d * bits / 8], low bits first."""
    per = 8 // bits
    c = np.asarray(codes, dtype=np.uint8)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per)).astype(np.uint32)
    out = np.zeros(c.shape[:-1], dtype=np.uint32)
    for k in range(per):
        out |= c[..., k] << (bits * k)
    return out.astype(np.uint8)


def unpack_rows(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of ``pack_rows``."""
    per = 8 // bits
    p = np.asarray(packed, dtype=np.uint8).astype(np.uint32)
    mask = (1 << bits) - 1
    parts = [((p >> (bits * k)) & mask) for k in range(per)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * per,)).astype(np.uint8)


# ----------------------------------------------------------------------------- the cache

class PagedCache:
    """Host copy of one layer's paged cache in the library's layout (see module docstring)."""

    def __init__(self, num_pages: int, kv_heads: int, page_size: int, head_dim: int, bits: int,
                 poison: bool = True):
        if page_size % 4:
            raise ValueError("page_size must be a multiple of 4")
        self.num_pages, self.kv_heads, self.page_size = num_pages, kv_heads, page_size
        self.head_dim, self.bits = head_dim, bits
        self.row = head_dim * bits // 8
        fill = 0xAA if poison else 0
        self.k_codes = np.full((num_pages, kv_heads, page_size, self.row), fill, dtype=np.uint8)
        self.v_codes = np.full((num_pages, kv_heads, page_size // 4, self.row, 4), fill, dtype=np.uint8)
        sz_fill = np.nan if poison else 0.0
        self.k_sz = np.full((num_pages, kv_heads, page_size, 2), sz_fill, dtype=np.float32)
        self.v_sz = np.full((num_pages, kv_heads, page_size, 2), sz_fill, dtype=np.float32)

    # token-level accessors: the one place that spells out the layout
    def write_token(self, page: int, off: int, head: int, k_row, k_scale, k_zero, v_row, v_scale, v_zero):
        self.k_codes[page, head, off, :] = k_row
        self.v_codes[page, head, off // 4, :, off % 4] = v_row
        self.k_sz[page, head, off] = (k_scale, k_zero)
        self.v_sz[page, head, off] = (v_scale, v_zero)

    def read_token(self, page: int, off: int, head: int):
        return (self.k_codes[page, head, off, :], self.k_sz[page, head, off],
                self.v_codes[page, head, off // 4, :, off % 4], self.v_sz[page, head, off])


def append(cache: PagedCache, k_bits: np.ndarray, v_bits: np.ndarray, slot_mapping: np.ndarray,
           hadamard_block: int, token_scale: int):
    """Rotate-quantize-append: tokens [T, kv_heads, d] of bf16 bits into ``cache`` at the slots.

    Returns the per-element diagnostics {'k_t', 'v_t'} (pre-rounding values, [T, H, d]) and
    the raw codes/scales/zeros per token, so tests can locate boundary elements.
    """
    t_n, h_n, d = k_bits.shape
    bits = cache.bits
    kc, ks, kz, kt = rotate_quantize(k_bits.reshape(t_n * h_n, d), hadamard_block, bits, token_scale)
    vc, vs, vz, vt = rotate_quantize(v_bits.reshape(t_n * h_n, d), hadamard_block, bits, token_scale)
    kp = pack_rows(kc, bits)
    vp = pack_rows(vc, bits)
    ps = cache.page_size
    for i in range(t_n):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        page, off = slot // ps, slot % ps
        for h in range(h_n):
            r = i * h_n + h
            cache.write_token(page, off, h, kp[r], ks[r], kz[r], vp[r], vs[r], vz[r])
    return {
        "k_codes": kc.reshape(t_n, h_n, d), "k_scale": ks.reshape(t_n, h_n), "k_zero": kz.reshape(t_n, h_n),
        "v_codes": vc.reshape(t_n, h_n, d), "v_scale": vs.reshape(t_n, h_n), "v_zero": vz.reshape(t_n, h_n),
        "k_t": kt.reshape(t_n, h_n, d), "v_t": vt.reshape(t_n, h_n, d),
    }


# ----------------------------------------------------------------------------- the read path

def gather_sequence(cache: PagedCache, block_table_row: np.ndarray, length: int, head: int):
    """Dequantized K and V (float64 [length, d], still in the rotated basis) of one sequence
    and KV head, read token by token through the page table."""
    d = cache.head_dim
    kh = np.empty((length, d), dtype=np.float64)
    vh = np.empty((length, d), dtype=np.float64)
    ps = cache.page_size
    for j in range(length):
        page = int(block_table_row[j // ps])
        k_row, k_sz, v_row, v_sz = cache.read_token(page, j % ps, head)
        kc = unpack_rows(k_row, cache.bits).astype(np.float64)
        vc = unpack_rows(v_row, cache.bits).astype(np.float64)
        kh[j] = kc * np.float64(k_sz[0]) + np.float64(k_sz[1])
        vh[j] = vc * np.float64(v_sz[0]) + np.float64(v_sz[1])
    return kh, vh


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale: float) -> np.ndarray:
    """softmax(softmax_scale * K q) V in float64 for one query vector; zeros if K is empty."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    s = softmax_scale * (np.asarray(k, dtype=np.float64) @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ np.asarray(v, dtype=np.float64)


def decode(cache: PagedCache, q_bits: np.ndarray, block_table: np.ndarray, context_lens: np.ndarray,
           num_kv_heads: int, hadamard_block: int, softmax_scale: float = 0.0, q_prerotated: int = 0,
           heads=None) -> np.ndarray:
    """Paged decode attention: float32 [B, Hq, d] output in the un-rotated basis.

    ``heads`` optionally restricts the work to a list of (b, q_head) pairs (other outputs
    are left as NaN) so that large workloads can be checked on a sample.
    """
    bsz, hq, d = q_bits.shape
    g = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(d)
    r = rotation_matrix(d, hadamard_block)
    out = np.full((bsz, hq, d), np.nan, dtype=np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(bsz) for h in range(hq)]
    cached = {}
    for b, h in todo:
        kvh = h // g
        length = int(context_lens[b])
        key = (b, kvh)
        if key not in cached:
            cached = {key: gather_sequence(cache, block_table[b], length, kvh)}
        kh, vh = cached[key]
        q = bf16_to_f32(q_bits[b, h]).astype(np.float64)
        qr = q if q_prerotated else r @ q
        o_rot = attend(qr, kh, vh, scale)
        out[b, h] = (r.T @ o_rot).astype(np.float32)
    return out


def multi_query_attention(cache: PagedCache, q_bits: np.ndarray, q_lens: np.ndarray, block_table: np.ndarray,
                          context_lens: np.ndarray, num_kv_heads: int, hadamard_block: int, softmax_scale: float = 0.0,
                          q_prerotated: int = 0, rows=None) -> np.ndarray:
    """Attention of several new tokens per sequence over the paged cache, causal (chunked prefill,
    speculative verification): sequence b's q_lens[b] queries are its last q_lens[b] tokens, already
    in the cache, so query j (0-based) sits at position context_lens[b] - q_lens[b] + j and attends
    to tokens 0 .. that position. q_bits bf16 [B, Q, Hq, d]; returns float32 [B, Q, Hq, d] in the
    un-rotated basis, zeros for j >= q_lens[b]. ``rows`` optionally restricts the work to (b, j, h)
    triples (others NaN)."""
    bsz, qmax, hq, d = q_bits.shape
    g = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(d)
    r = rotation_matrix(d, hadamard_block)
    out = np.full((bsz, qmax, hq, d), np.nan if rows is not None else 0.0, dtype=np.float32)
    todo = rows if rows is not None else [(b, j, h) for b in range(bsz) for j in range(int(q_lens[b]))
                                          for h in range(hq)]
    cached = {}
    for b, j, h in todo:
        if j >= int(q_lens[b]):
            out[b, j, h] = 0.0
            continue
        kvh = h // g
        length = int(context_lens[b])
        key = (b, kvh)
        if key not in cached:
            cached = {key: gather_sequence(cache, block_table[b], length, kvh)}
        kh, vh = cached[key]
        n = length - int(q_lens[b]) + j + 1          # causal: the query's own position included
        q = bf16_to_f32(q_bits[b, j, h]).astype(np.float64)
        qr = q if q_prerotated else r @ q
        out[b, j, h] = (r.T @ attend(qr, kh[:n], vh[:n], scale)).astype(np.float32)
    return out


def dequant_page(cache: PagedCache, page: int, hadamard_block: int, unrotate: int, tensor: str = "k") -> np.ndarray:
    """All tokens of one page of the K (``tensor="k"``) or V half, dequantized:
    float32 [kv_heads, page_size, d].

    code * scale + zero is formed in float64 and rounded once to float32; with
    ``unrotate`` the rows are mapped back by R^T (float64, rounded once to float32).
    """
    d = cache.head_dim
    out = np.empty((cache.kv_heads, cache.page_size, d), dtype=np.float32)
    r = rotation_matrix(d, hadamard_block)
    for h in range(cache.kv_heads):
        for off in range(cache.page_size):
            k_row, k_sz, v_row, v_sz = cache.read_token(page, off, h)
            row, sz = (k_row, k_sz) if tensor == "k" else (v_row, v_sz)
            c = unpack_rows(row, cache.bits).astype(np.float64)
            x = c * np.float64(sz[0]) + np.float64(sz[1])
            if unrotate:
                x = r.T @ x
            out[h, off] = x.astype(np.float32)
    return out


# ----------------------------------------------------------------------------- bf16 baseline

class PagedCacheBF16:
    """Unquantized bf16 paged cache of the baseline decode (the kind of cache a BF16 split
    decode such as FlashDecoding-v2, the OScaR abstract's point of comparison, reads):

      K  uint16 (bf16 bits) [num_pages][kv_heads][page_size][head_dim]          token-major rows
      V  uint16 (bf16 bits) [num_pages][kv_heads][page_size / 16][head_dim][16]  channel-major
         inside each run of 16 tokens: V of token t, channel c at [.., t // 16, c, t % 16]
    """

    def __init__(self, num_pages, kv_heads, page_size, head_dim, poison=True):
        self.num_pages, self.kv_heads, self.page_size, self.head_dim = num_pages, kv_heads, page_size, head_dim
        fill = 0x7FC0 if poison else 0  # bf16 NaN
        self.k = np.full((num_pages, kv_heads, page_size, head_dim), fill, dtype=np.uint16)
        self.v = np.full((num_pages, kv_heads, page_size // 16, head_dim, 16), fill, dtype=np.uint16)

    def write_token(self, page, off, head, k_row, v_row):
        self.k[page, head, off, :] = k_row
        self.v[page, head, off // 16, :, off % 16] = v_row

    def read_token(self, page, off, head):
        return self.k[page, head, off, :], self.v[page, head, off // 16, :, off % 16]


def append_bf16(cache: PagedCacheBF16, k_bits: np.ndarray, v_bits: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Copy bf16 K/V [T, H, d] to their slots unchanged (negative or out-of-pool slots skipped)."""
    ps = cache.page_size
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= cache.num_pages * ps:
            continue
        for h in range(cache.kv_heads):
            cache.write_token(int(slot // ps), int(slot % ps), h, k_bits[t, h], v_bits[t, h])


def decode_bf16(cache: PagedCacheBF16, q_bits: np.ndarray, block_table: np.ndarray, context_lens: np.ndarray,
                num_kv_heads: int, softmax_scale: float = 0.0, heads=None) -> np.ndarray:
    """Paged decode attention over the bf16 cache (no rotation, no quantization): float32
    [B, Hq, d]; query head h reads KV head h // (Hq / H_kv); a sequence of length 0 gives zeros."""
    bsz, hq, d = q_bits.shape
    g = hq // num_kv_heads
    scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(d)
    ps = cache.page_size
    out = np.full((bsz, hq, d), np.nan, dtype=np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(bsz) for h in range(hq)]
    for b, h in todo:
        kvh = h // g
        n = int(context_lens[b])
        ks = np.zeros((n, d), dtype=np.float64)
        vs = np.zeros((n, d), dtype=np.float64)
        for j in range(n):
            kr, vr = cache.read_token(int(block_table[b, j // ps]), j % ps, kvh)
            ks[j] = bf16_to_f32(kr)
            vs[j] = bf16_to_f32(vr)
        out[b, h] = attend(bf16_to_f32(q_bits[b, h]), ks, vs, scale).astype(np.float32)
    return out


# ----------------------------------------------------------------------------- per-channel pages
# The per-channel reading of OScaR (OScaR abstract on the openalex page: rotation and per-token
# scaling make the per-channel quantization paradigm work under extreme compression; zhichai.net
# summary, "The OScaR Framework": V-hat = Quant(S (R V))). Each token is rotated (y = R x) and
# divided by its own scale s (the token's RMS, as in the token-wise variant); the normalised tokens
# u = y / s of one page then share one asymmetric (scale, zero) pair per channel. A page is
# quantized once all its tokens exist; the tokens of a sequence's unfinished last page stay in
# bf16 (the residual window) and are attended as they are.
#
# Layout (caller-owned arrays):
#   K codes  [num_pages][kv_heads][page_size][row]          as in the token-wise cache
#   V codes  [num_pages][kv_heads][page_size / 4][row][4]   as in the token-wise cache
#   K/V s    float32 [num_pages][kv_heads][page_size]         per-token scale
#   K/V cp   float32 [num_pages][kv_heads][2][head_dim]       {scale[d], zero[d]} per channel
#   tail     bf16 bits [batch][page_size][kv_heads][head_dim] the residual window of each sequence


def quantize_channels(u: np.ndarray, bits: int):
    """Per-channel asymmetric quantization of float32 u [T, d] over its T tokens.

    Returns (codes uint8 [T, d], scale float32 [d], zero float32 [d], t float64 [T, d]), t being
    the pre-rounding value (u - min) / scale in float64 from the float32 operands. Same rule as
    the token-wise quantizer, with the minimum and maximum taken down each channel.
    """
    u = np.asarray(u, dtype=np.float32)
    qmax = np.float32(2 ** bits - 1)
    mn = u.min(axis=0)
    mx = u.max(axis=0)
    scale = (mx - mn) / qmax                            # float32 subtract, IEEE divide
    live = scale != 0
    safe = np.where(live, scale, np.float32(1.0))
    tf = (u - mn[None, :]) / safe[None, :]              # float32, IEEE divide
    codes = np.clip(np.rint(tf), 0, qmax).astype(np.uint8)
    codes[:, ~live] = 0
    t = (u.astype(np.float64) - mn[None, :].astype(np.float64)) / safe[None, :].astype(np.float64)
    t[:, ~live] = 0.0
    return codes, scale.astype(np.float32), mn.astype(np.float32), t


class PagedCachePC:
    """Host copy of a per-channel cache (layout in the comment above)."""

    def __init__(self, num_pages: int, kv_heads: int, page_size: int, head_dim: int, bits: int,
                 poison: bool = True):
        if page_size % 4:
            raise ValueError("page_size must be a multiple of 4")
        self.num_pages, self.kv_heads, self.page_size = num_pages, kv_heads, page_size
        self.head_dim, self.bits = head_dim, bits
        self.row = head_dim * bits // 8
        fill = 0xAA if poison else 0
        f_fill = np.nan if poison else 0.0
        self.k_codes = np.full((num_pages, kv_heads, page_size, self.row), fill, dtype=np.uint8)
        self.v_codes = np.full((num_pages, kv_heads, page_size // 4, self.row, 4), fill, dtype=np.uint8)
        self.k_s = np.full((num_pages, kv_heads, page_size), f_fill, dtype=np.float32)
        self.v_s = np.full((num_pages, kv_heads, page_size), f_fill, dtype=np.float32)
        self.k_cp = np.full((num_pages, kv_heads, 2, head_dim), f_fill, dtype=np.float32)
        self.v_cp = np.full((num_pages, kv_heads, 2, head_dim), f_fill, dtype=np.float32)

    def write_page(self, page: int, head: int, kc, ks, kcp, vc, vs, vcp):
        """Codes [ps, d], token scales [ps] and (scale, zero) [2, d] of K and V of one page-head."""
        kp = pack_rows(kc, self.bits)
        vp = pack_rows(vc, self.bits)
        self.k_codes[page, head] = kp
        for t in range(self.page_size):
            self.v_codes[page, head, t // 4, :, t % 4] = vp[t]
        self.k_s[page, head] = ks
        self.v_s[page, head] = vs
        self.k_cp[page, head] = kcp
        self.v_cp[page, head] = vcp

    def read_page(self, page: int, head: int, tensor: str):
        """(codes uint8 [ps, d], token scales [ps], (scale, zero) [2, d]) of one page-head."""
        if tensor == "k":
            packed = self.k_codes[page, head]
            return unpack_rows(packed, self.bits), self.k_s[page, head], self.k_cp[page, head]
        packed = self.v_codes[page, head].transpose(0, 2, 1).reshape(self.page_size, self.row)
        return unpack_rows(packed, self.bits), self.v_s[page, head], self.v_cp[page, head]


def quantize_page_pc(x_bits: np.ndarray, b: int, bits: int):
    """One page-head of one tensor: bf16 bits [ps, d] -> (codes [ps, d], s [ps], cp [2, d], t).

    y = R x per token (float32), s = RMS(y) per token, u = y / s (float32, IEEE divide), then the
    per-channel quantizer over the page's tokens.
    """
    return quantize_rotated_page_pc(rotate_f32(bf16_to_f32(x_bits), b), bits)


def quantize_rotated_page_pc(y: np.ndarray, bits: int):
    """``quantize_page_pc`` from the rotated tokens y (float32 [ps, d]) on."""
    s = token_rms(y)
    u = y / s[:, None]
    codes, sc, zr, t = quantize_channels(u, bits)
    return codes, s, np.stack([sc, zr]).astype(np.float32), t


def write_pages_pc(cache: PagedCachePC, k_bits: np.ndarray, v_bits: np.ndarray, page_ids: np.ndarray,
                   hadamard_block: int):
    """Quantize whole pages: input page i is tokens i * ps .. i * ps + ps - 1 of k_bits / v_bits
    ([n * ps, kv_heads, d] bf16 bits) and goes to cache page page_ids[i] (negative: skipped).
    Returns the pre-rounding values {'k_t', 'v_t'} [n, kv_heads, ps, d] for boundary checks."""
    ps, h_n, d = cache.page_size, cache.kv_heads, cache.head_dim
    n = len(page_ids)
    k_t = np.zeros((n, h_n, ps, d))
    v_t = np.zeros((n, h_n, ps, d))
    # every token rotated in one pass (rows are independent), then page by page
    yk = rotate_f32(bf16_to_f32(k_bits[:n * ps].reshape(-1, d)), hadamard_block).reshape(n, ps, h_n, d)
    yv = rotate_f32(bf16_to_f32(v_bits[:n * ps].reshape(-1, d)), hadamard_block).reshape(n, ps, h_n, d)
    for i in range(n):
        page = int(page_ids[i])
        for h in range(h_n):
            kc, ks, kcp, kt = quantize_rotated_page_pc(yk[i, :, h], cache.bits)
            vc, vs, vcp, vt = quantize_rotated_page_pc(yv[i, :, h], cache.bits)
            k_t[i, h], v_t[i, h] = kt, vt
            if page >= 0:
                cache.write_page(page, h, kc, ks, kcp, vc, vs, vcp)
    return {"k_t": k_t, "v_t": v_t}


def dequant_page_pc(cache: PagedCachePC, page: int, head: int, tensor: str) -> np.ndarray:
    """float64 [ps, d] in the rotated basis: s_t (code * scale_c + zero_c)."""
    codes, s, cp = cache.read_page(page, head, tensor)
    u = codes.astype(np.float64) * cp[0].astype(np.float64)[None, :] + cp[1].astype(np.float64)[None, :]
    return u * s.astype(np.float64)[:, None]


def decode_pc(cache: PagedCachePC, q_bits: np.ndarray, block_table: np.ndarray, context_lens: np.ndarray,
              tail_k_bits: np.ndarray, tail_v_bits: np.ndarray, num_kv_heads: int, hadamard_block: int,
              softmax_scale: float = 0.0, heads=None) -> np.ndarray:
    """Decode attention over a per-channel cache plus the residual window, float32 [B, Hq, d].

    Sequence b of length L has L // ps complete pages (block_table[b][0 ..]) and L % ps tokens in
    tail[b][0 ..]. The pages are dequantized and rotated back (R is its own inverse), the tail is
    used as given; then softmax attention of the bf16 query over all L tokens.
    """
    bsz, hq, d = q_bits.shape
    g = hq // num_kv_heads
    ps = cache.page_size
    scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(d)
    r = rotation_matrix(d, hadamard_block)
    out = np.full((bsz, hq, d), np.nan, dtype=np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(bsz) for h in range(hq)]
    cached = {}
    for b, h in todo:
        kvh = h // g
        length = int(context_lens[b])
        if (b, kvh) not in cached:
            n_full, n_tail = length // ps, length % ps
            ks, vs = [], []
            for j in range(n_full):
                page = int(block_table[b, j])
                ks.append(dequant_page_pc(cache, page, kvh, "k") @ r)   # rows: (R k)^T R = k^T
                vs.append(dequant_page_pc(cache, page, kvh, "v") @ r)
            ks.append(bf16_to_f32(tail_k_bits[b, :n_tail, kvh]).astype(np.float64))
            vs.append(bf16_to_f32(tail_v_bits[b, :n_tail, kvh]).astype(np.float64))
            cached[(b, kvh)] = (np.concatenate(ks, axis=0), np.concatenate(vs, axis=0))
        kk, vv = cached[(b, kvh)]
        q = bf16_to_f32(q_bits[b, h]).astype(np.float64)
        out[b, h] = attend(q, kk, vv, scale).astype(np.float32)
    return out

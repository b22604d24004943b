"""Seeded synthetic inputs for the rotated low-bit paged KV cache.

This module draws numbers and nothing else: bf16 K/V/Q values with the shapes and value
distributions of the workloads described on the pages (outlier channels, log-normal
per-token norms), physical page assignments, page tables, slot mappings and context
lengths. It holds no step of the method (no rotation, no quantization, no attention), so
the CPU oracle and the HIP path can both consume exactly the same inputs without sharing
any arithmetic.

Workload shapes (head_dim 128, page size 16 throughout):
  * ``tiny``       - 1 sequence, 8/8 heads, 512 tokens, Hadamard block 32, INT4.
  * ``llama3_8b``  - 16 sequences, 32/8 heads (GQA 4), 4096 tokens, block 128, INT4.
  * ``sweep_b{B}`` - B sequences of the Llama-3-8B layer shape, ragged lengths
                     uniform in [512, 8192], block 64, INT4.
  * ``llama2_70b`` - 4 sequences, 64/8 heads (GQA 8), 32768 tokens, block 128, INT4,
                     80 independent layer caches.
  * ``oscar_int2`` - 32 sequences, 28/4 heads (GQA 7), 16384 tokens, block 128, INT2
                     with the per-token scaling step, chunked prefill in 512-token
                     chunks that start inside partially filled pages.

Distribution recipe (all draws from independent sub-streams of ``SeedSequence(seed)``):
  K and V entries are N(0, 1); a fixed set of ``num_outliers`` channels (same for every
  head and layer) is multiplied by ``outlier_scale``; every token's vector is then
  multiplied by a factor drawn from LogNormal(0, ``lognorm_sigma``), drawn separately for
  K and V and shared by that token's KV heads; the result is rounded to bf16 (round to
  nearest even). Queries are N(0, 1) rounded to bf16.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16

# Sub-stream indices of SeedSequence(seed).spawn(...)
_S_OUTLIER, _S_KVAL, _S_KNORM, _S_VVAL, _S_VNORM, _S_Q, _S_PAGES, _S_LENS, _S_CHUNK, _S_NEW = range(10)
_N_STREAMS = 10


@dataclass(frozen=True)
class Shape:
    """Sizes and distribution parameters of one synthetic workload."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    context_lens: tuple          # tokens already in the cache per sequence (prefill length)
    hadamard_block: int
    bits: int
    token_scale: int
    outlier_scale: float
    num_outliers: int
    lognorm_sigma: float
    seed: int
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE
    layers: int = 1
    chunk: int = 0               # >0: prefill arrives in chunks of this many tokens
    spare_page_frac: float = 0.01

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        """Longest attended length in a decode step (prefill plus the new token)."""
        return max(self.context_lens) + 1

    def with_(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


def _sweep_lens(batch: int, seed: int) -> tuple:
    ss = np.random.SeedSequence(seed).spawn(_N_STREAMS)
    rng = np.random.Generator(np.random.PCG64(ss[_S_LENS]))
    return tuple(int(x) for x in rng.integers(512, 8192, size=batch, endpoint=True))


def config(name: str, **overrides) -> Shape:
    """Return the workload called ``name`` (see the module docstring), with overrides."""
    if name == "tiny":
        s = Shape(name, 1, 8, 8, (512,), 32, 4, 0, 10.0, 4, 1.0, seed=1000)
    elif name == "llama3_8b":
        s = Shape(name, 16, 32, 8, (4096,) * 16, 128, 4, 0, 10.0, 4, 1.0, seed=1001)
    elif name.startswith("sweep_b"):
        b = int(name[len("sweep_b"):])
        s = Shape(name, b, 32, 8, _sweep_lens(b, 1002), 64, 4, 0, 10.0, 4, 1.0, seed=1002)
    elif name == "llama2_70b":
        s = Shape(name, 4, 64, 8, (32768,) * 4, 128, 4, 0, 20.0, 4, 1.5, seed=1003, layers=80)
    elif name == "oscar_int2":
        s = Shape(name, 32, 28, 4, (16384,) * 32, 128, 2, 1, 1.0, 0, 2.0, seed=1004, chunk=512)
    else:
        raise KeyError(f"unknown workload {name!r}")
    return s.with_(**overrides) if overrides else s


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(_N_STREAMS)]


# ----------------------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + (0x7FFF + ((u >> 16) & 1))) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- values

def outlier_channels(shape: Shape) -> np.ndarray:
    if shape.num_outliers == 0:
        return np.zeros(0, dtype=np.int64)
    rng = _streams(shape.seed)[_S_OUTLIER]
    return np.sort(rng.choice(shape.head_dim, shape.num_outliers, replace=False))


def _draw_values(shape: Shape, val_rng, norm_rng, n_tokens: int) -> np.ndarray:
    x = val_rng.standard_normal((n_tokens, shape.num_kv_heads, shape.head_dim), dtype=np.float32)
    ch = outlier_channels(shape)
    if ch.size:
        x[:, :, ch] *= np.float32(shape.outlier_scale)
    f = norm_rng.lognormal(0.0, shape.lognorm_sigma, size=n_tokens).astype(np.float32)
    x *= f[:, None, None]
    return f32_to_bf16_bits(x)


def draw_kv(shape: Shape, n_tokens: int, layer: int = 0, stream: str = "prefill"):
    """K and V bf16 bits, each [n_tokens, num_kv_heads, head_dim] (uint16).

    ``stream`` selects independent draws for the prefill tokens and for decode tokens;
    ``layer`` gives each layer its own values.
    """
    base = shape.seed * 1_000_003 + layer * 7919 + (0 if stream == "prefill" else 104729)
    st = _streams(base)
    k = _draw_values(shape, st[_S_KVAL], st[_S_KNORM], n_tokens)
    v = _draw_values(shape, st[_S_VVAL], st[_S_VNORM], n_tokens)
    return k, v


def draw_q(shape: Shape, layer: int = 0) -> np.ndarray:
    """Decode queries, bf16 bits [batch, num_q_heads, head_dim]."""
    rng = _streams(shape.seed * 1_000_003 + layer * 7919 + 31)[_S_Q]
    q = rng.standard_normal((shape.batch, shape.num_q_heads, shape.head_dim), dtype=np.float32)
    return f32_to_bf16_bits(q)


# ----------------------------------------------------------------------------- pages

@dataclass
class PagePlan:
    """Physical page assignment for one layer's cache."""
    num_pages: int
    block_table: np.ndarray      # int32 [batch, max_pages_per_seq], -1 where unused
    capacity: np.ndarray         # int64 [batch] tokens each sequence may hold


def plan_pages(shape: Shape, extra_tokens: int = 1, layer: int = 0) -> PagePlan:
    """Give every sequence enough pages for its prefill plus ``extra_tokens`` decode tokens,
    drawing physical page ids as a seeded random permutation of the pool (1 % spare pages)."""
    ps = shape.page_size
    lens = np.asarray(shape.context_lens, dtype=np.int64)
    cap = lens + extra_tokens
    need = (cap + ps - 1) // ps
    total = int(need.sum())
    num_pages = total + int(np.ceil(total * shape.spare_page_frac))
    rng = _streams(shape.seed * 1_000_003 + layer * 7919 + 17)[_S_PAGES]
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = int(need.max()) if len(need) else 0
    bt = np.full((shape.batch, max(max_pages, 1)), -1, dtype=np.int32)
    pos = 0
    for b in range(shape.batch):
        n = int(need[b])
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return PagePlan(num_pages, bt, cap)


def identity_pages(shape: Shape, extra_tokens: int = 1) -> PagePlan:
    """Same capacity as ``plan_pages`` but with pages handed out in order (page table = iota)."""
    ps = shape.page_size
    lens = np.asarray(shape.context_lens, dtype=np.int64)
    cap = lens + extra_tokens
    need = (cap + ps - 1) // ps
    total = int(need.sum())
    max_pages = int(need.max()) if len(need) else 0
    bt = np.full((shape.batch, max(max_pages, 1)), -1, dtype=np.int32)
    pos = 0
    for b in range(shape.batch):
        n = int(need[b])
        bt[b, :n] = np.arange(pos, pos + n, dtype=np.int32)
        pos += n
    return PagePlan(total, bt, cap)


def slots_for_positions(plan: PagePlan, page_size: int, seq: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Slot (physical page * page_size + offset) of token position ``pos`` of sequence ``seq``."""
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    page = plan.block_table[seq, pos // page_size].astype(np.int64)
    return page * page_size + pos % page_size


def prefill_order(shape: Shape):
    """(seq, pos) of every prefill token, sequence by sequence, positions ascending."""
    lens = np.asarray(shape.context_lens, dtype=np.int64)
    seq = np.repeat(np.arange(shape.batch, dtype=np.int64), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    pos = np.arange(int(lens.sum()), dtype=np.int64) - np.repeat(starts, lens)
    return seq, pos


def chunk_schedule(shape: Shape):
    """Chunked prefill: a list of (seq, pos) arrays, one per append call.

    Every sequence first receives r_b ~ U{1..15} tokens, so that all later chunks of
    ``shape.chunk`` tokens start inside a partially filled page; the remaining tokens then
    arrive one chunk per sequence per call, round-robin over the sequences.
    """
    assert shape.chunk > 0
    rng = _streams(shape.seed)[_S_CHUNK]
    lens = np.asarray(shape.context_lens, dtype=np.int64)
    first = np.minimum(rng.integers(1, 15, size=shape.batch, endpoint=True), lens)
    calls = []
    seqs = np.arange(shape.batch, dtype=np.int64)
    calls.append((np.repeat(seqs, first), np.concatenate([np.arange(f) for f in first])))
    done = first.copy()
    while (done < lens).any():
        s_list, p_list = [], []
        for b in range(shape.batch):
            n = int(min(shape.chunk, lens[b] - done[b]))
            if n > 0:
                s_list.append(np.full(n, b, dtype=np.int64))
                p_list.append(np.arange(done[b], done[b] + n, dtype=np.int64))
                done[b] += n
        calls.append((np.concatenate(s_list), np.concatenate(p_list)))
    return calls


def decode_positions(shape: Shape):
    """(seq, pos) of the one new token each sequence appends in a decode step."""
    return np.arange(shape.batch, dtype=np.int64), np.asarray(shape.context_lens, dtype=np.int64)


def shuffled_slot_mapping(rng_seed: int, n: int, num_slots: int) -> np.ndarray:
    """``n`` distinct random slots out of ``num_slots`` (for placement tests)."""
    rng = np.random.Generator(np.random.PCG64(rng_seed))
    return rng.choice(num_slots, n, replace=False).astype(np.int64)


# ----------------------------------------------------------------------------- device draws

def draw_kv_device(shape: Shape, n_tokens: int, device, layer: int = 0, stream: str = "prefill"):
    """Same recipe as ``draw_kv`` (N(0, 1) entries, the workload's outlier channels scaled,
    per-token LogNormal(0, sigma) factors drawn separately for K and V, bf16 rounding), drawn
    with torch's generator on ``device``: for timing runs whose inputs are too large to draw on
    the host. The values differ from ``draw_kv``'s (another generator); the distribution is the
    same. Returns two bf16 tensors [n_tokens, num_kv_heads, head_dim]."""
    import torch

    seed = (shape.seed * 1_000_003 + layer * 7919 + (0 if stream == "prefill" else 104729)) % (2 ** 63)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    ch = torch.as_tensor(outlier_channels(shape), device=device, dtype=torch.long)
    out = []
    for _ in range(2):
        x = torch.randn((n_tokens, shape.num_kv_heads, shape.head_dim), generator=g, device=device,
                        dtype=torch.float32)
        if ch.numel():
            x[:, :, ch] *= shape.outlier_scale
        f = torch.empty(n_tokens, device=device, dtype=torch.float32).log_normal_(0.0, shape.lognorm_sigma, generator=g)
        x *= f[:, None, None]
        out.append(x.to(torch.bfloat16))
    return out[0], out[1]


def draw_q_device(shape: Shape, device, layer: int = 0):
    """Decode queries drawn on ``device`` (N(0, 1), bf16), [batch, num_q_heads, head_dim]."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((shape.seed * 1_000_003 + layer * 7919 + 31) % (2 ** 63))
    return torch.randn((shape.batch, shape.num_q_heads, shape.head_dim), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)

"""Python binding of libkvq (ctypes). Argument marshalling only: every step of the write and
read paths runs in the library's HIP kernels. PyTorch provides device memory and streams.

The library must have been built (``python -m paged_decode_attention_amd.build``); there is
no fallback: if it is missing, or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")
HEAD_DIM = 128

KVQ_OK, KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = range(6)

EXPORTS = ("kvq_abi_version", "kvq_status_string", "kvq_rotate_quantize_append",
           "kvq_paged_decode_workspace_size", "kvq_paged_decode_attention", "kvq_dequant_page",
           "kvq_bf16_cache_write", "kvq_paged_decode_attention_bf16", "kvq_decode_step",
           "kvq_paged_prefill_workspace_size", "kvq_paged_prefill_attention", "kvq_pc_write_pages",
           "kvq_pc_decode_workspace_size", "kvq_pc_decode_attention", "kvq_paged_decode_bf16_workspace_size",
           "kvq_paged_decode_attention_noalloc", "kvq_paged_prefill_kernel")


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None
_c = ctypes
_p, _i32, _i64, _f32, _sz = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_float, _c.c_size_t


def lib() -> ctypes.CDLL:
    """Load libkvq.so (once) and declare its signatures; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_decode_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.kvq_abi_version.restype = _i32
    L.kvq_abi_version.argtypes = []
    L.kvq_status_string.restype = _c.c_char_p
    L.kvq_status_string.argtypes = [_i32]
    L.kvq_rotate_quantize_append.restype = _i32
    L.kvq_rotate_quantize_append.argtypes = [
        _p, _p, _i64, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p]
    L.kvq_paged_decode_workspace_size.restype = _sz
    L.kvq_paged_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    L.kvq_paged_decode_attention.restype = _i32
    L.kvq_paged_decode_attention.argtypes = [
        _p, _i32, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        _p, _p, _sz, _i32, _p]
    L.kvq_paged_decode_attention_noalloc.restype = _i32
    L.kvq_paged_decode_attention_noalloc.argtypes = [
        _p, _i32, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        _p, _i32, _p]
    L.kvq_dequant_page.restype = _i32
    L.kvq_dequant_page.argtypes = [_p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p]
    L.kvq_paged_prefill_kernel.restype = _i32
    L.kvq_paged_prefill_kernel.argtypes = [_i32, _i32, _i32, _i32]
    L.kvq_paged_prefill_workspace_size.restype = _sz
    L.kvq_paged_prefill_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
    L.kvq_paged_prefill_attention.restype = _i32
    L.kvq_paged_prefill_attention.argtypes = [
        _p, _i32, _p, _i32, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        _p, _p, _sz, _i32, _p]
    L.kvq_decode_step.restype = _i32
    L.kvq_decode_step.argtypes = [
        _p, _i32, _p, _p, _i64, _i64, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
        _i32, _f32, _p, _p, _sz, _i32, _p]
    L.kvq_bf16_cache_write.restype = _i32
    L.kvq_bf16_cache_write.argtypes = [_p, _p, _i64, _i64, _i64, _i32, _i32, _p, _p, _p, _i32, _i32, _p]
    L.kvq_paged_decode_bf16_workspace_size.restype = _sz
    L.kvq_paged_decode_bf16_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    L.kvq_paged_decode_attention_bf16.restype = _i32
    L.kvq_paged_decode_attention_bf16.argtypes = [
        _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _sz, _i32, _p]
    L.kvq_pc_write_pages.restype = _i32
    L.kvq_pc_write_pages.argtypes = [
        _p, _p, _i64, _i64, _i32, _p, _i32, _i32, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p]
    L.kvq_pc_decode_workspace_size.restype = _sz
    L.kvq_pc_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    L.kvq_pc_decode_attention.restype = _i32
    L.kvq_pc_decode_attention.argtypes = [
        _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        _p, _p, _sz, _i32, _p]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().kvq_abi_version())


def _check(status: int, where: str):
    if status != KVQ_OK:
        raise KVQError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _own_workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace allocated for one call on ``stream``: the allocation is made with
    that stream current, so the caching allocator does not hand its memory to another stream's
    work while the call's kernels may still use it."""
    if stream is None:
        return decode_workspace(nbytes, device)
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        return decode_workspace(nbytes, device)


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _workspace(workspace):
    """(pointer, bytes) of a caller's workspace: a contiguous device tensor of any dtype, or None."""
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device (cuda/hip) tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


# ----------------------------------------------------------------------------- cache

@dataclass
class PagedKVCache:
    """One layer's paged cache in the library's layout (four device tensors)."""
    k_codes: torch.Tensor   # uint8 [P, H, ps, row]
    v_codes: torch.Tensor   # uint8 [P, H, ps/4, row, 4]
    k_sz: torch.Tensor      # float32 [P, H, ps, 2]
    v_sz: torch.Tensor      # float32 [P, H, ps, 2]
    bits: int

    @staticmethod
    def empty(num_pages: int, num_kv_heads: int, page_size: int, bits: int, device="cuda",
              head_dim: int = HEAD_DIM) -> "PagedKVCache":
        row = head_dim * bits // 8
        return PagedKVCache(
            torch.empty((num_pages, num_kv_heads, page_size, row), dtype=torch.uint8, device=device),
            torch.empty((num_pages, num_kv_heads, page_size // 4, row, 4), dtype=torch.uint8, device=device),
            torch.empty((num_pages, num_kv_heads, page_size, 2), dtype=torch.float32, device=device),
            torch.empty((num_pages, num_kv_heads, page_size, 2), dtype=torch.float32, device=device),
            bits)

    @property
    def num_pages(self) -> int:
        return self.k_codes.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k_codes.shape[1]

    @property
    def page_size(self) -> int:
        return self.k_codes.shape[2]

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k_codes, self.v_codes, self.k_sz, self.v_sz))

    def _check_layout(self):
        p, h, ps, row = self.k_codes.shape
        if row != HEAD_DIM * self.bits // 8 or tuple(self.v_codes.shape) != (p, h, ps // 4, row, 4):
            raise ValueError("cache tensors do not match the documented layout")
        if tuple(self.k_sz.shape) != (p, h, ps, 2) or tuple(self.v_sz.shape) != (p, h, ps, 2):
            raise ValueError("scale/zero tensors do not match the documented layout")
        for t in (self.k_codes, self.v_codes, self.k_sz, self.v_sz):
            if not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous")


# ----------------------------------------------------------------------------- write path

def rotate_quantize_append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, cache: PagedKVCache,
                           hadamard_block: int, token_scale: int = 0, stream=None) -> None:
    """kvq_rotate_quantize_append on bf16 k, v [T, H, 128] (head vectors contiguous) and int64 slots [T]."""
    cache._check_layout()
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or t.shape[1] != cache.num_kv_heads or t.shape[2] != HEAD_DIM or t.stride(2) != 1 \
                or t.stride(1) != HEAD_DIM:
            raise ValueError(f"{name} must be [T, {cache.num_kv_heads}, {HEAD_DIM}] with contiguous heads")
    if k.shape[0] != v.shape[0] or slot_mapping.shape != (k.shape[0],) or not slot_mapping.is_contiguous():
        raise ValueError("k, v and slot_mapping disagree on the number of tokens")
    st = lib().kvq_rotate_quantize_append(
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16), k.stride(0), v.stride(0), k.shape[0],
        cache.num_kv_heads, HEAD_DIM, _dev(slot_mapping, "slot_mapping", torch.int64),
        _dev(cache.k_codes, "k_codes", torch.uint8), _dev(cache.v_codes, "v_codes", torch.uint8),
        _dev(cache.k_sz, "k_sz", torch.float32), _dev(cache.v_sz, "v_sz", torch.float32),
        cache.num_pages, cache.page_size, hadamard_block, cache.bits, token_scale, _stream(stream))
    _check(st, "kvq_rotate_quantize_append")


# ----------------------------------------------------------------------------- read path

def decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_context_len: int, page_size: int,
                          pages_per_split: int = 0) -> int:
    return int(lib().kvq_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, HEAD_DIM, max_context_len,
                                                       page_size, pages_per_split))


def decode_workspace(nbytes: int, device) -> torch.Tensor:
    """A decode workspace of ``nbytes`` (its contents do not matter to the library)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def decode_bf16_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_context_len: int,
                               page_size: int, pages_per_split: int = 0) -> int:
    return int(lib().kvq_paged_decode_bf16_workspace_size(batch, num_q_heads, num_kv_heads, HEAD_DIM,
                                                            max_context_len, page_size, pages_per_split))


def paged_decode_attention(q: torch.Tensor, cache: PagedKVCache, block_table: torch.Tensor,
                           context_lens: torch.Tensor, max_context_len: int, hadamard_block: int,
                           softmax_scale: float = 0.0, q_prerotated: int = 0, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, pages_per_split: int = 0,
                           stream=None) -> torch.Tensor:
    """kvq_paged_decode_attention: q bf16 [B, Hq, 128] -> float32 [B, Hq, 128] (un-rotated)."""
    cache._check_layout()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    bsz, hq, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != bsz or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (bsz, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, 128] float32 tensor")
    need = decode_workspace_size(bsz, hq, cache.num_kv_heads, max_context_len, cache.page_size, pages_per_split)
    if workspace is None and need > 0:
        workspace = _own_workspace(need, q.device, stream)
    ws_ptr, ws_bytes = _workspace(workspace)
    st = lib().kvq_paged_decode_attention(
        _dev(q, "q", torch.bfloat16), q_prerotated,
        _dev(cache.k_codes, "k_codes", torch.uint8), _dev(cache.v_codes, "v_codes", torch.uint8),
        _dev(cache.k_sz, "k_sz", torch.float32), _dev(cache.v_sz, "v_sz", torch.float32),
        cache.num_pages, cache.page_size, _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), max_context_len, bsz, hq, cache.num_kv_heads, HEAD_DIM,
        hadamard_block, cache.bits, float(softmax_scale), _dev(out, "out", torch.float32), ws_ptr, ws_bytes,
        pages_per_split, _stream(stream))
    _check(st, "kvq_paged_decode_attention")
    return out


# Bytes of the fixed scratch behind kvq_paged_decode_attention_noalloc (KVQ_DECODE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20


def paged_decode_attention_noalloc(q: torch.Tensor, cache: PagedKVCache, block_table: torch.Tensor,
                                   context_lens: torch.Tensor, max_context_len: int, hadamard_block: int,
                                   out: torch.Tensor, softmax_scale: float = 0.0, q_prerotated: int = 0,
                                   pages_per_split: int = 0, stream=None) -> torch.Tensor:
    """kvq_paged_decode_attention_noalloc: the decode with its split partials in the library's fixed
    scratch; nothing is allocated (``out`` is the caller's). Calls that overlap on one GPU race."""
    cache._check_layout()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    bsz, hq, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != bsz or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    if tuple(out.shape) != (bsz, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, 128] float32 tensor")
    st = lib().kvq_paged_decode_attention_noalloc(
        _dev(q, "q", torch.bfloat16), q_prerotated,
        _dev(cache.k_codes, "k_codes", torch.uint8), _dev(cache.v_codes, "v_codes", torch.uint8),
        _dev(cache.k_sz, "k_sz", torch.float32), _dev(cache.v_sz, "v_sz", torch.float32),
        cache.num_pages, cache.page_size, _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), max_context_len, bsz, hq, cache.num_kv_heads, HEAD_DIM,
        hadamard_block, cache.bits, float(softmax_scale), _dev(out, "out", torch.float32), pages_per_split,
        _stream(stream))
    _check(st, "kvq_paged_decode_attention_noalloc")
    return out


def prefill_workspace_size(batch: int, max_q_len: int, num_q_heads: int, num_kv_heads: int, max_context_len: int,
                           page_size: int, pages_per_split: int = 0) -> int:
    return int(lib().kvq_paged_prefill_workspace_size(batch, max_q_len, num_q_heads, num_kv_heads, HEAD_DIM,
                                                       max_context_len, page_size, pages_per_split))


def prefill_kernel(batch: int, max_q_len: int, num_q_heads: int, num_kv_heads: int) -> int:
    """kvq_paged_prefill_kernel: 1 large-chunk kernel, 0 split kernel, -1 rejected sizes."""
    return int(lib().kvq_paged_prefill_kernel(batch, max_q_len, num_q_heads, num_kv_heads))


def paged_prefill_attention(q: torch.Tensor, q_lens: torch.Tensor, cache: PagedKVCache, block_table: torch.Tensor,
                            context_lens: torch.Tensor, max_context_len: int, hadamard_block: int,
                            softmax_scale: float = 0.0, q_prerotated: int = 0, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, pages_per_split: int = 0,
                            stream=None) -> torch.Tensor:
    """kvq_paged_prefill_attention: q bf16 [B, Q, Hq, 128], q_lens int32 [B] -> float32 [B, Q, Hq, 128]."""
    cache._check_layout()
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Q, Hq, 128] tensor")
    bsz, qmax, hq, _ = q.shape
    if q_lens.shape != (bsz,) or not q_lens.is_contiguous():
        raise ValueError("q_lens must be a contiguous [B] int32 tensor")
    if block_table.dim() != 2 or block_table.shape[0] != bsz or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    if out is None:
        out = torch.empty((bsz, qmax, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (bsz, qmax, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Q, Hq, 128] float32 tensor")
    need = prefill_workspace_size(bsz, qmax, hq, cache.num_kv_heads, max_context_len, cache.page_size,
                                  pages_per_split)
    if prefill_kernel(bsz, qmax, hq, cache.num_kv_heads) == 1:
        need = 0  # the large-chunk kernel leaves the workspace untouched
    if workspace is None and need > 0:
        workspace = _own_workspace(need, q.device, stream)
    ws_ptr, ws_bytes = _workspace(workspace)
    st = lib().kvq_paged_prefill_attention(
        _dev(q, "q", torch.bfloat16), q_prerotated, _dev(q_lens, "q_lens", torch.int32), qmax,
        _dev(cache.k_codes, "k_codes", torch.uint8), _dev(cache.v_codes, "v_codes", torch.uint8),
        _dev(cache.k_sz, "k_sz", torch.float32), _dev(cache.v_sz, "v_sz", torch.float32),
        cache.num_pages, cache.page_size, _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), max_context_len, bsz, hq, cache.num_kv_heads, HEAD_DIM,
        hadamard_block, cache.bits, float(softmax_scale), _dev(out, "out", torch.float32), ws_ptr, ws_bytes,
        pages_per_split, _stream(stream))
    _check(st, "kvq_paged_prefill_attention")
    return out


def decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache: PagedKVCache,
                block_table: torch.Tensor, context_lens: torch.Tensor, max_context_len: int, hadamard_block: int,
                token_scale: int = 0, softmax_scale: float = 0.0, q_prerotated: int = 0,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, pages_per_split: int = 0,
                stream=None) -> torch.Tensor:
    """kvq_decode_step: append k_new, v_new [B, H, 128] (bf16) at position context_lens[b] - 1 of each
    sequence, then attend; returns float32 [B, Hq, 128]."""
    cache._check_layout()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    bsz, hq, _ = q.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 3 or t.shape[0] != bsz or t.shape[1] != cache.num_kv_heads or t.shape[2] != HEAD_DIM \
                or t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
            raise ValueError(f"{name} must be [B, {cache.num_kv_heads}, {HEAD_DIM}] with contiguous heads")
    if block_table.dim() != 2 or block_table.shape[0] != bsz or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (bsz, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, 128] float32 tensor")
    need = decode_workspace_size(bsz, hq, cache.num_kv_heads, max_context_len, cache.page_size, pages_per_split)
    if workspace is None and need > 0:
        workspace = _own_workspace(need, q.device, stream)
    ws_ptr, ws_bytes = _workspace(workspace)
    st = lib().kvq_decode_step(
        _dev(q, "q", torch.bfloat16), q_prerotated, _dev(k_new, "k_new", torch.bfloat16),
        _dev(v_new, "v_new", torch.bfloat16), k_new.stride(0), v_new.stride(0),
        _dev(cache.k_codes, "k_codes", torch.uint8), _dev(cache.v_codes, "v_codes", torch.uint8),
        _dev(cache.k_sz, "k_sz", torch.float32), _dev(cache.v_sz, "v_sz", torch.float32),
        cache.num_pages, cache.page_size, _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), max_context_len, bsz, hq, cache.num_kv_heads, HEAD_DIM,
        hadamard_block, cache.bits, token_scale, float(softmax_scale), _dev(out, "out", torch.float32), ws_ptr,
        ws_bytes, pages_per_split, _stream(stream))
    _check(st, "kvq_decode_step")
    return out


def dequant_page(cache: PagedKVCache, tensor: str, page: int, hadamard_block: int, unrotate: int = 0,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_dequant_page for the K (``tensor="k"``) or V half: float32 [H, ps, 128]."""
    cache._check_layout()
    codes, sz = (cache.k_codes, cache.k_sz) if tensor == "k" else (cache.v_codes, cache.v_sz)
    if out is None:
        out = torch.empty((cache.num_kv_heads, cache.page_size, HEAD_DIM), dtype=torch.float32,
                          device=codes.device)
    st = lib().kvq_dequant_page(_dev(codes, "codes", torch.uint8), _dev(sz, "sz", torch.float32),
                                0 if tensor == "k" else 1, page, cache.num_pages, cache.num_kv_heads,
                                cache.page_size, HEAD_DIM, hadamard_block, cache.bits, unrotate,
                                _dev(out, "out", torch.float32), _stream(stream))
    _check(st, "kvq_dequant_page")
    return out


# ----------------------------------------------------------------------------- bf16 baseline

@dataclass
class PagedKVCacheBF16:
    """Unquantized bf16 cache of the baseline decode (two device tensors of bf16)."""
    k: torch.Tensor   # bfloat16 [P, H, ps, 128]
    v: torch.Tensor   # bfloat16 [P, H, ps/16, 128, 16]

    @staticmethod
    def empty(num_pages: int, num_kv_heads: int, page_size: int, device="cuda") -> "PagedKVCacheBF16":
        return PagedKVCacheBF16(
            torch.empty((num_pages, num_kv_heads, page_size, HEAD_DIM), dtype=torch.bfloat16, device=device),
            torch.empty((num_pages, num_kv_heads, page_size // 16, HEAD_DIM, 16), dtype=torch.bfloat16, device=device))

    @property
    def num_pages(self) -> int:
        return self.k.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def page_size(self) -> int:
        return self.k.shape[2]

    def _check_layout(self):
        p, h, ps, d = self.k.shape
        if d != HEAD_DIM or tuple(self.v.shape) != (p, h, ps // 16, HEAD_DIM, 16):
            raise ValueError("bf16 cache tensors do not match the documented layout")
        if not (self.k.is_contiguous() and self.v.is_contiguous()):
            raise ValueError("cache tensors must be contiguous")


def bf16_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, cache: PagedKVCacheBF16,
                     stream=None) -> None:
    """kvq_bf16_cache_write on bf16 k, v [T, H, 128] (contiguous heads) and int64 slots [T]."""
    cache._check_layout()
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or t.shape[1] != cache.num_kv_heads or t.shape[2] != HEAD_DIM or t.stride(2) != 1 \
                or t.stride(1) != HEAD_DIM:
            raise ValueError(f"{name} must be [T, {cache.num_kv_heads}, {HEAD_DIM}] with contiguous heads")
    if k.shape[0] != v.shape[0] or slot_mapping.shape != (k.shape[0],) or not slot_mapping.is_contiguous():
        raise ValueError("k, v and slot_mapping disagree on the number of tokens")
    st = lib().kvq_bf16_cache_write(
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16), k.stride(0), v.stride(0), k.shape[0],
        cache.num_kv_heads, HEAD_DIM, _dev(slot_mapping, "slot_mapping", torch.int64),
        _dev(cache.k, "k_cache", torch.bfloat16), _dev(cache.v, "v_cache", torch.bfloat16), cache.num_pages,
        cache.page_size, _stream(stream))
    _check(st, "kvq_bf16_cache_write")


def paged_decode_attention_bf16(q: torch.Tensor, cache: PagedKVCacheBF16, block_table: torch.Tensor,
                                context_lens: torch.Tensor, max_context_len: int, softmax_scale: float = 0.0,
                                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                pages_per_split: int = 0, stream=None) -> torch.Tensor:
    """kvq_paged_decode_attention_bf16: q bf16 [B, Hq, 128] -> float32 [B, Hq, 128]."""
    cache._check_layout()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    bsz, hq, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != bsz or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (bsz, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, 128] float32 tensor")
    need = decode_bf16_workspace_size(bsz, hq, cache.num_kv_heads, max_context_len, cache.page_size,
                                      pages_per_split)
    if workspace is None and need > 0:
        workspace = _own_workspace(need, q.device, stream)
    ws_ptr, ws_bytes = _workspace(workspace)
    st = lib().kvq_paged_decode_attention_bf16(
        _dev(q, "q", torch.bfloat16), _dev(cache.k, "k_cache", torch.bfloat16), _dev(cache.v, "v_cache", torch.bfloat16),
        cache.num_pages, cache.page_size, _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), max_context_len, bsz, hq, cache.num_kv_heads, HEAD_DIM,
        float(softmax_scale), _dev(out, "out", torch.float32), ws_ptr, ws_bytes, pages_per_split, _stream(stream))
    _check(st, "kvq_paged_decode_attention_bf16")
    return out


# ----------------------------------------------------------------------------- per-channel pages

@dataclass
class PagedKVCachePC:
    """Per-channel cache of the OScaR per-channel reading (six device tensors): codes as in
    ``PagedKVCache``, a float32 scale per token and a float32 (scale, zero) per channel per page-head."""
    k_codes: torch.Tensor   # uint8 [P, H, ps, row]
    v_codes: torch.Tensor   # uint8 [P, H, ps/4, row, 4]
    k_s: torch.Tensor       # float32 [P, H, ps]
    v_s: torch.Tensor       # float32 [P, H, ps]
    k_cp: torch.Tensor      # float32 [P, H, 2, 128] = {scale[128], zero[128]}
    v_cp: torch.Tensor      # float32 [P, H, 2, 128]
    bits: int

    @staticmethod
    def empty(num_pages: int, num_kv_heads: int, page_size: int, bits: int, device="cuda") -> "PagedKVCachePC":
        row = HEAD_DIM * bits // 8
        u8, f32 = torch.uint8, torch.float32
        return PagedKVCachePC(
            torch.empty((num_pages, num_kv_heads, page_size, row), dtype=u8, device=device),
            torch.empty((num_pages, num_kv_heads, page_size // 4, row, 4), dtype=u8, device=device),
            torch.empty((num_pages, num_kv_heads, page_size), dtype=f32, device=device),
            torch.empty((num_pages, num_kv_heads, page_size), dtype=f32, device=device),
            torch.empty((num_pages, num_kv_heads, 2, HEAD_DIM), dtype=f32, device=device),
            torch.empty((num_pages, num_kv_heads, 2, HEAD_DIM), dtype=f32, device=device), bits)

    @property
    def num_pages(self) -> int:
        return self.k_codes.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k_codes.shape[1]

    @property
    def page_size(self) -> int:
        return self.k_codes.shape[2]

    def _check_layout(self):
        p, h, ps, row = self.k_codes.shape
        if row != HEAD_DIM * self.bits // 8 or tuple(self.v_codes.shape) != (p, h, ps // 4, row, 4) \
                or tuple(self.k_s.shape) != (p, h, ps) or tuple(self.v_s.shape) != (p, h, ps) \
                or tuple(self.k_cp.shape) != (p, h, 2, HEAD_DIM) or tuple(self.v_cp.shape) != (p, h, 2, HEAD_DIM):
            raise ValueError("per-channel cache tensors do not match the documented layout")
        for t in (self.k_codes, self.v_codes, self.k_s, self.v_s, self.k_cp, self.v_cp):
            if not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous")


def pc_write_pages(k: torch.Tensor, v: torch.Tensor, page_ids: torch.Tensor, cache: PagedKVCachePC,
                   hadamard_block: int, stream=None) -> None:
    """kvq_pc_write_pages: k, v bf16 [n * ps, H, 128] (contiguous heads), input page i = tokens
    i * ps .. i * ps + ps - 1, written to cache page page_ids[i] (int32 [n])."""
    cache._check_layout()
    ps = cache.page_size
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or t.shape[1] != cache.num_kv_heads or t.shape[2] != HEAD_DIM or t.stride(2) != 1 \
                or t.stride(1) != HEAD_DIM or t.shape[0] % ps:
            raise ValueError(f"{name} must be [n * {ps}, {cache.num_kv_heads}, {HEAD_DIM}] with contiguous heads")
    n = k.shape[0] // ps
    if v.shape[0] != k.shape[0] or page_ids.shape != (n,) or not page_ids.is_contiguous():
        raise ValueError("k, v and page_ids disagree on the number of pages")
    st = lib().kvq_pc_write_pages(
        _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16), k.stride(0), v.stride(0), n,
        _dev(page_ids, "page_ids", torch.int32), cache.num_kv_heads, HEAD_DIM,
        _dev(cache.k_codes, "k_codes", torch.uint8), _dev(cache.v_codes, "v_codes", torch.uint8),
        _dev(cache.k_s, "k_s", torch.float32), _dev(cache.v_s, "v_s", torch.float32),
        _dev(cache.k_cp, "k_cp", torch.float32), _dev(cache.v_cp, "v_cp", torch.float32),
        cache.num_pages, ps, hadamard_block, cache.bits, _stream(stream))
    _check(st, "kvq_pc_write_pages")


def pc_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_context_len: int, page_size: int,
                             pages_per_split: int = 0) -> int:
    return int(lib().kvq_pc_decode_workspace_size(batch, num_q_heads, num_kv_heads, HEAD_DIM, max_context_len,
                                                  page_size, pages_per_split))


def pc_decode_attention(q: torch.Tensor, cache: PagedKVCachePC, block_table: torch.Tensor,
                        context_lens: torch.Tensor, max_context_len: int, tail_k: torch.Tensor, tail_v: torch.Tensor,
                        hadamard_block: int, softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, pages_per_split: int = 0, stream=None) -> torch.Tensor:
    """kvq_pc_decode_attention: q bf16 [B, Hq, 128]; sequence b's context_lens[b] // ps complete pages
    come from block_table[b], its context_lens[b] % ps newest tokens from tail_k / tail_v
    (bf16 [B, ps, H, 128]). Returns float32 [B, Hq, 128]."""
    cache._check_layout()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    bsz, hq, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != bsz or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] int32 tensor")
    tail_shape = (bsz, cache.page_size, cache.num_kv_heads, HEAD_DIM)
    for name, t in (("tail_k", tail_k), ("tail_v", tail_v)):
        if tuple(t.shape) != tail_shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {list(tail_shape)} bf16 tensor")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (bsz, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, 128] float32 tensor")
    if workspace is None:
        workspace = _own_workspace(pc_decode_workspace_size(bsz, hq, cache.num_kv_heads, max_context_len,
                                                            cache.page_size, pages_per_split), q.device, stream)
    st = lib().kvq_pc_decode_attention(
        _dev(q, "q", torch.bfloat16), _dev(cache.k_codes, "k_codes", torch.uint8),
        _dev(cache.v_codes, "v_codes", torch.uint8), _dev(cache.k_s, "k_s", torch.float32),
        _dev(cache.v_s, "v_s", torch.float32), _dev(cache.k_cp, "k_cp", torch.float32),
        _dev(cache.v_cp, "v_cp", torch.float32), cache.num_pages, cache.page_size,
        _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), max_context_len,
        _dev(tail_k, "tail_k", torch.bfloat16), _dev(tail_v, "tail_v", torch.bfloat16), bsz, hq,
        cache.num_kv_heads, HEAD_DIM, hadamard_block, cache.bits, float(softmax_scale), _dev(out, "out", torch.float32),
        *_workspace(workspace), pages_per_split, _stream(stream))
    _check(st, "kvq_pc_decode_attention")
    return out

"""ctypes binding of libkvq_stream.so (include/kvq_stream.h): streaming probes that measure the
HBM bandwidth a launch of a given shape reaches when it only moves bytes. Measurement support:
the KV-cache path never calls it."""
from __future__ import annotations

import ctypes
import os

import torch

_LIB = None
_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_stream.so")
EXPORTS = ("kvq_stream_probe",)


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build it with python -m paged_decode_attention_amd.build")
        L = ctypes.CDLL(_PATH)
        L.kvq_stream_probe.restype = ctypes.c_int32
        L.kvq_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
        _LIB = L
    return _LIB


def probe(src: torch.Tensor | None, dst: torch.Tensor | None, rows: int, read_units: int, write_units: int,
          grid_blocks: int, block_threads: int, sink: torch.Tensor, stream=None, src_offset: int = 0,
          dst_offset: int = 0, layout: int = 0) -> None:
    """One launch: ``rows`` rows of ``read_units`` 16-byte loads from ``src`` (from byte
    ``src_offset``) and ``write_units`` 16-byte stores to ``dst`` (from ``dst_offset``); layout 0
    interleaves them within each wave, layout 1 splits the workgroups into readers and writers."""
    need_r, need_w = rows * read_units * 16, rows * write_units * 16
    if read_units and (src is None or src_offset + need_r > src.numel() * src.element_size()):
        raise ValueError("src too small for the rows read")
    if write_units and (dst is None or dst_offset + need_w > dst.numel() * dst.element_size()):
        raise ValueError("dst too small for the rows written")
    s = torch.cuda.current_stream() if stream is None else stream
    sp = (src.data_ptr() + src_offset) if read_units else None
    dp = (dst.data_ptr() + dst_offset) if write_units else None
    st = lib().kvq_stream_probe(sp, dp, rows, read_units, write_units, layout, grid_blocks, block_threads,
                                0x9E3779B9, sink.data_ptr(), s.cuda_stream)
    if st != 0:
        raise RuntimeError(f"kvq_stream_probe failed with status {st}")

"""Rotated low-bit paged KV cache for AMD Instinct MI355X (gfx950).

* ``kvq``        - ctypes binding of libkvq.so (the HIP kernels behind a C ABI, include/kvq.h)
* ``workloads``  - seeded synthetic inputs shaped like the workloads on the pages
* ``build``      - compiles libkvq.so in-tree with hipcc
"""

"""Helpers for the GPU parity tests: moving seeded inputs to the device, reading a device
cache back into the documented layout, building large host caches from the oracle, and the
agreement rules for codes, scales/zeros and attention outputs.

Agreement rules (derived from the arithmetic of the method):
  * codes and page placement: bit-exact, except an element whose oracle pre-rounding value
    t = (u - min) / scale lies within 1e-5 of a half-integer may differ by exactly one code
    step (the HIP butterflies and the oracle's dense matmul round in a different order); the
    number of such elements must stay below 1e-6 of all compared elements;
  * scale: |s_gpu - s_ref| <= 1e-6 * max(s_ref, M / qmax), zero: |z_gpu - z_ref| <= 1e-6 * M,
    with M = max(|min|, |max|) of the token's (scaled) range;
  * attention output: relative L2 error <= 2e-3 per (sequence, query head) vector.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvq_oracle as O
from paged_decode_attention_amd import kvq
from paged_decode_attention_amd import workloads as W

BOUNDARY_BAND = 1e-5
MISMATCH_RATE = 1e-6
SZ_RTOL = 1e-6
ATTN_RTOL = 2e-3


# ----------------------------------------------------------------------------- device I/O

def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def poisoned_device_cache(num_pages, kv_heads, page_size, bits, device="cuda") -> kvq.PagedKVCache:
    c = kvq.PagedKVCache.empty(num_pages, kv_heads, page_size, bits, device=device)
    c.k_codes.fill_(0xAA)
    c.v_codes.fill_(0xAA)
    c.k_sz.fill_(float("nan"))
    c.v_sz.fill_(float("nan"))
    return c


def upload_cache(host: O.PagedCache, device="cuda") -> kvq.PagedKVCache:
    return kvq.PagedKVCache(to_dev(host.k_codes, device), to_dev(host.v_codes, device), to_dev(host.k_sz, device),
                            to_dev(host.v_sz, device), host.bits)


def download_cache(dev: kvq.PagedKVCache) -> O.PagedCache:
    p, h, ps, row = dev.k_codes.shape
    c = O.PagedCache(p, h, ps, 128, dev.bits, poison=False)
    c.k_codes[:] = dev.k_codes.cpu().numpy()
    c.v_codes[:] = dev.v_codes.cpu().numpy()
    c.k_sz[:] = dev.k_sz.cpu().numpy()
    c.v_sz[:] = dev.v_sz.cpu().numpy()
    return c


# ----------------------------------------------------------------------------- layout views

def cache_codes(c: O.PagedCache):
    """(K codes, V codes) as uint8 [P, H, ps, D], read with the documented byte layout."""
    p, h, ps, row = c.k_codes.shape
    k = O.unpack_rows(c.k_codes, c.bits)
    v_rows = c.v_codes.transpose(0, 1, 2, 4, 3).reshape(p, h, ps, row)
    v = O.unpack_rows(v_rows, c.bits)
    return k, v


def host_cache_from_oracle(k_bits, v_bits, slots, num_pages, page_size, hb, bits, token_scale):
    """A host cache holding exactly what ``O.append`` would write, with the placement done by
    vectorised numpy scatter (for workloads too large for the oracle's per-token loop).
    ``test_parity_helpers.py`` checks it against ``O.append`` on small inputs."""
    t_n, h_n, d = k_bits.shape
    c = O.PagedCache(num_pages, h_n, page_size, d, bits)
    live = slots >= 0
    page = slots[live] // page_size
    off = slots[live] % page_size
    diag = {}
    for name, x, codes_arr, sz_arr in (("k", k_bits, c.k_codes, c.k_sz), ("v", v_bits, c.v_codes, c.v_sz)):
        cq, sc, zr, t = O.rotate_quantize(x.reshape(t_n * h_n, d), hb, bits, token_scale)
        rows = O.pack_rows(cq, bits).reshape(t_n, h_n, -1)[live]           # [n, H, row]
        for h in range(h_n):
            if name == "k":
                codes_arr[page, h, off, :] = rows[:, h]
            else:
                codes_arr[page, h, off // 4, :, off % 4] = rows[:, h]
            sz_arr[page, h, off, 0] = sc.reshape(t_n, h_n)[live, h]
            sz_arr[page, h, off, 1] = zr.reshape(t_n, h_n)[live, h]
        diag[name] = (cq.reshape(t_n, h_n, d), sc.reshape(t_n, h_n), zr.reshape(t_n, h_n), t.reshape(t_n, h_n, d))
    return c, diag


# ----------------------------------------------------------------------------- agreement

def check_codes(gpu_codes: np.ndarray, ref_codes: np.ndarray, t: np.ndarray, what: str):
    """Codes must be equal except near-boundary elements off by one; returns the mismatch count."""
    diff = gpu_codes.astype(np.int16) - ref_codes.astype(np.int16)
    bad = diff != 0
    n_bad = int(bad.sum())
    if n_bad:
        frac = np.abs(t[bad] - np.floor(t[bad]) - 0.5)
        assert np.all(np.abs(diff[bad]) == 1), f"{what}: code differs by more than one step"
        assert np.all(frac < BOUNDARY_BAND), f"{what}: mismatch away from a rounding boundary (|frac-0.5| max {frac.max()})"
    allowed = int(MISMATCH_RATE * gpu_codes.size)
    assert n_bad <= allowed, f"{what}: {n_bad} boundary mismatches among {gpu_codes.size} elements (allowed {allowed})"
    return n_bad


def check_scale_zero(gpu_s, gpu_z, ref_s, ref_z, bits, what: str):
    qmax = 2 ** bits - 1
    ref_s = ref_s.astype(np.float64)
    ref_z = ref_z.astype(np.float64)
    m = np.maximum(np.abs(ref_z), np.abs(ref_z + qmax * ref_s))
    ds = np.abs(gpu_s.astype(np.float64) - ref_s)
    dz = np.abs(gpu_z.astype(np.float64) - ref_z)
    assert np.all(ds <= SZ_RTOL * np.maximum(ref_s, m / qmax)), f"{what}: scale off by up to {ds.max()}"
    assert np.all(dz <= SZ_RTOL * m), f"{what}: zero off by up to {dz.max()}"


def rel_l2(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error per vector along the last axis (absolute error where the reference is 0)."""
    num = np.linalg.norm(gpu.astype(np.float64) - ref.astype(np.float64), axis=-1)
    den = np.linalg.norm(ref.astype(np.float64), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def check_attention(gpu: np.ndarray, ref: np.ndarray, what: str, heads=None):
    if heads is not None:
        idx = tuple(np.array(heads).T)
        gpu, ref = gpu[idx], ref[idx]
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    e = rel_l2(gpu, ref)
    assert e.max() <= ATTN_RTOL, f"{what}: worst rel-L2 {e.max():.3e} (global {np.linalg.norm(gpu - ref) / np.linalg.norm(ref):.3e})"
    return float(e.max())

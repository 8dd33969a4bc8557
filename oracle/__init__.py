"""fp64 CPU oracle for scaled dot-product attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (``transformer_attention_04_amd``)
never imports it, and this package imports nothing from the product path.

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double, libm ``exp``):
the explicit definition of Eq. A on the page "Shape-Aware Attention" (section
"Inspiration"), softmax(Q K^T * scale) V, one query row at a time, with the
causal rule "key j visible to query i iff j <= kv_len - S_q + i".  This module
only marshals numpy arrays into it.

``kv_append`` is the K/V cache append of the streaming use, a numpy slice
assignment (no arithmetic).

Parity status of each function is stated where it is tested (``tests/
test_oracle_pins.py``): the attention function is pinned by closed forms,
invariants, a library special case (torch CPU float64 SDPA with an explicit
mask) and 50-digit brute force; ``kv_append`` by an element-by-element loop,
two appends against one, and raw bit patterns; neither is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORACLE_ERRORS = {1: "bad argument", 2: "bad row list", 3: "out of memory"}


def build(out: str = _LIB, src: str = _SRC) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE order kept)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first only if nothing is built) and return the ctypes handle."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    f = lib.oracle_attn_f64
    i64 = ctypes.c_int64
    f.argtypes = [ctypes.c_void_p] * 4 + [i64] * 5 + [ctypes.c_int, ctypes.c_double, i64,
                                                   ctypes.c_void_p, i64, ctypes.c_int]
    f.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def max_threads() -> int:
    return int(load().oracle_max_threads())


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor on the CPU
        import torch
        x = x.detach()
        if x.dtype != torch.float32:
            x = x.to(torch.float32)  # bf16/fp16 -> fp32 is exact
        x = x.contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def attention(q, k, v, *, causal: bool = False, scale: float | None = None,
              kv_len: int | None = None, rows=None, threads: int = 0,
              lib=None) -> np.ndarray:
    """Eq. A in fp64.  q: [B,H,S_q,D], k/v: [B,H,S_kv,D] (float32 values, or torch
    CPU tensors of any float dtype, promoted exactly).  scale None -> 1/sqrt(D).
    kv_len None -> S_kv.  rows: optional query-row indices computed for every
    (b,h); the result then has shape [B,H,len(rows),D].  Returns float64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B,H,S,D]")
    B, H, S_q, D = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    S_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    if kv_len is None:
        kv_len = S_kv
    rows_arr = None
    n_rows = S_q
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        n_rows = rows_arr.size
    o = np.empty((B, H, n_rows, D), dtype=np.float64)
    lib = lib or load()
    rc = lib.oracle_attn_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                             B, H, S_q, S_kv, D, int(bool(causal)), float(scale), int(kv_len),
                             rows_arr.ctypes.data if rows_arr is not None else None,
                             int(n_rows), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_f64: {ORACLE_ERRORS.get(rc, rc)}")
    return o


def kv_append(k_cache, v_cache, k_new, v_new, kv_len):
    """The K/V cache append of a stream of query windows against a growing
    key/value cache (page "Roofline", section "How we built it"): copies of
    the caches [B, H, S_cap, D] whose rows [kv_len, kv_len + n) of every
    (b, h) are the new rows [B, H, n, D]; every other row is unchanged.  The
    plain definition, a slice assignment on numpy arrays of any dtype (bit
    patterns are copied as they are)."""
    k_out, v_out = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    n = k_new.shape[2]
    if kv_len < 0 or kv_len + n > k_out.shape[2]:
        raise ValueError("kv_len + n exceeds the cache capacity")
    k_out[:, :, kv_len:kv_len + n] = k_new
    v_out[:, :, kv_len:kv_len + n] = v_new
    return k_out, v_out

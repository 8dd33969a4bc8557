"""fp64 CPU oracle for scaled dot-product attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (``transformer_attention_04_amd``)
never imports it, and this package imports nothing from the product path.

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double, libm ``exp``):
the explicit definition of the attention equation on the page "Shape-Aware
Attention" (section "Inspiration"), softmax(Q K^T * scale) V, one query row at a time, with the
causal rule "key j visible to query i iff j <= kv_len - S_q + i".  This module
only marshals numpy arrays into it.

``attention_varlen`` is the attention equation for a batch of sequences of different lengths
padded to one K/V capacity: per sequence, the same function on its own K/V
prefix (a slice), with the bottom-right causal rule of that sequence's length
and zeros for a query row that sees no key.  ``kv_append`` is the K/V cache
append of the streaming use, a numpy slice assignment (no arithmetic).
``qkv_projection`` is the fused Q/K/V projection upstream of attention: one
matrix product with the stacked weights, in fp64, split into heads.

Parity status of each function is stated where it is tested (``tests/
test_oracle_pins.py``): the attention function is pinned by closed forms,
invariants, a library special case (torch CPU float64 SDPA with an explicit
mask) and 50-digit brute force; ``attention_varlen`` by SDPA with a
per-sequence mask, padding that holds NaN, empty and single-key rows and
batch permutations; ``kv_append`` by an element-by-element loop, two appends
against one, and raw bit patterns; ``qkv_projection`` by brute-force loops,
identity and zero-input closed forms, head permutations and linearity; none is
"parity unpinned".
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
    """The attention equation in fp64.  q: [B,H,S_q,D], k/v: [B,H,S_kv,D] (float32 values, or torch
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


def attention_varlen(q, k, v, kv_lens, *, causal: bool = False, scale: float | None = None,
                     threads: int = 0, lib=None) -> np.ndarray:
    """The attention equation per sequence of a padded batch (key padding).  q: [B,H,S_q,D],
    k/v: [B,H,S_kv,D]; sequence b attends only to its first L_b K/V rows,
    L_b = kv_lens[b] clamped into [0, S_kv].  Causal: query row i of sequence
    b sits at position L_b - S_q + i (bottom-right, as in ``attention``) and
    sees keys j <= that position.  A row that sees no key -- L_b = 0, or a
    causal row with L_b - S_q + i < 0 -- is zero: the pages define the softmax
    only over a non-empty set, and zero is the empty weighted sum.  Each
    sequence is ``attention`` on its slice k[b, :, :L_b] and on its query rows
    from i0 = max(0, S_q - L_b) on (the rows that see a key; the slice keeps
    their positions, since L_b - (S_q - i0) + (i - i0) = L_b - S_q + i).
    Returns float64 [B,H,S_q,D]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, S_q, D = q.shape
    S_kv = k.shape[2]
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    if lens.size != B:
        raise ValueError(f"kv_lens has {lens.size} values for a batch of {B}")
    o = np.zeros((B, H, S_q, D), dtype=np.float64)
    for b in range(B):
        L = int(min(max(int(lens[b]), 0), S_kv))
        if L == 0:
            continue
        i0 = max(0, S_q - L) if causal else 0
        if i0 == S_q:
            continue
        o[b:b + 1, :, i0:] = attention(q[b:b + 1, :, i0:], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                       causal=causal, scale=scale, threads=threads, lib=lib)
    return o


def qkv_projection(x, w, bias, H: int):
    """The fused Q/K/V projection (page "Roofline", sections "What it does" and
    "How we built it": the three projections of a layer's input as one larger
    kernel).  x: [B, S, d] with d = 64*H; w: [3d, d], the three projection
    weights stacked in the layout of a linear layer (output feature o is row
    o; rows [0, d) give Q, [d, 2d) K, [2d, 3d) V; inside each, head h is
    features [64h, 64h + 64)); bias: [3d] or None.  y = x w^T + bias in fp64;
    returns (q, k, v), each float64 [B, H, S, 64] with q[b, h, s, e] =
    y[b, s, 64h + e] and likewise k, v from the next two thirds."""
    x = np.asarray(_f32(x), dtype=np.float64)
    w = np.asarray(_f32(w), dtype=np.float64)
    B, S, d = x.shape
    if d != 64 * H or w.shape != (3 * d, d):
        raise ValueError(f"shapes x{x.shape} w{w.shape} do not match H={H}, head size 64")
    y = x.reshape(B * S, d) @ w.T
    if bias is not None:
        y = y + np.asarray(_f32(bias), dtype=np.float64).reshape(1, 3 * d)
    y = y.reshape(B, S, 3, H, 64)
    return tuple(np.ascontiguousarray(y[:, :, j].transpose(0, 2, 1, 3)) for j in range(3))


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

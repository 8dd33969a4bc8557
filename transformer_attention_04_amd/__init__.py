"""Python binding of the MI355X fused attention forward library (libattn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h.  torch supplies device
memory and the current stream.  There is no fallback: if the library is not
built, importing this package raises.

    attn_fwd(q, k, v, causal=False, scale=None)            -> o   (alias fwd)
    attn_fwd_chunked(q, k, v, chunk, kv_len=None, ...)       -> o   (alias fwd_chunked)
    attn_fwd_varlen(q, k, v, kv_lens, causal=False, ...)     -> o
    attn_fwd_splitkv(q, k, v, causal=False, n_split=0, ...)  -> o
    attn_fwd_splitkv_noalloc(q, k, v, out, causal=False, ...) -> out
    attn_kv_append(k_cache, v_cache, k_new, v_new, kv_len)   -> kv_len + n
    attn_qkv_proj(x, w, bias=None)                           -> (q, k, v)
    attn_strerror(status)                                    -> str

q: [B, H, S_q, 64]; k, v: [B, H, S_kv, 64]; all contiguous, same dtype
(float32, float16 or bfloat16) and same CUDA (HIP) device.  scale=None means
1/sqrt(64) (the attention equation of page "Shape-Aware Attention", section
"Inspiration").
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
STATUS = {
    0: "ATTN_OK", 1: "ATTN_E_NULL", 2: "ATTN_E_SHAPE", 3: "ATTN_E_DTYPE", 4: "ATTN_E_SCALE",
    5: "ATTN_E_CAUSAL", 6: "ATTN_E_CHUNK", 7: "ATTN_E_ALIGN", 8: "ATTN_E_DEVICE",
    9: "ATTN_E_HIP", 10: "ATTN_E_OVERLAP", 11: "ATTN_E_SPLIT", 12: "ATTN_E_WORKSPACE",
}
globals().update({name: code for code, name in STATUS.items()})
NOALLOC_SCRATCH_BYTES = 16 << 20  # ATTN_NOALLOC_SCRATCH_BYTES in include/attn.h
EXPORTS = ("attn_fwd", "attn_fwd_chunked", "attn_fwd_varlen", "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc",
           "attn_splitkv_workspace_bytes",
           "attn_splitkv_choose", "attn_kv_append", "attn_qkv_proj", "attn_strerror", "attn_sched_rows",
           "attn_sched_grid", "attn_sched_tile")


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run transformer_attention_04_amd/build.py "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    # torch ships its own HIP runtime under the same soname as the system one
    # this library links.  Loaded after torch, the library binds to torch's
    # copy; loaded first, it would pull in the system runtime and torch would
    # then load its own as well: two runtimes in one process, and torch's
    # streams and memory would be foreign to this library's calls.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, ctypes.c_float, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_chunked.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, ctypes.c_float, i, vp, i, i]
    lib.attn_fwd_chunked.restype = i
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, ctypes.c_float, i, vp, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, ctypes.c_float, i, vp, i, i, vp,
                                     ctypes.c_size_t]
    lib.attn_fwd_splitkv.restype = i
    lib.attn_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, ctypes.c_float, i, vp, i, i]
    lib.attn_fwd_splitkv_noalloc.restype = i
    lib.attn_splitkv_workspace_bytes.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_splitkv_workspace_bytes.restype = i
    lib.attn_splitkv_choose.argtypes = [i, i, i, i, i, ctypes.POINTER(i)]
    lib.attn_splitkv_choose.restype = i
    lib.attn_qkv_proj.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.attn_qkv_proj.restype = i
    lib.attn_kv_append.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.attn_kv_append.restype = i
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_sched_rows.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.attn_sched_rows.restype = i
    lib.attn_sched_grid.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(i)]
    lib.attn_sched_grid.restype = i
    lib.attn_sched_tile.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.attn_sched_tile.restype = i
    return lib


lib = _load()


def attn_strerror(status: int) -> str:
    return lib.attn_strerror(int(status)).decode()


_codes = None


def _dtype_code(t) -> int:
    global _codes
    if _codes is None:
        torch = _t()
        _codes = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
    c = _codes.get(t.dtype)
    if c is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return c


def _check(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, D], got {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, S_q, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, H, S_q, k.shape[2], D


_torch = None
_raw_stream = None


def _t():
    """torch, imported on first use (the library itself does not need it)."""
    global _torch, _raw_stream
    if _torch is None:
        import torch
        _torch = torch
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    return _torch


def _stream_ptr(device, stream):
    torch = _t()
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _call(fn, device, *args):
    """Call into the library with `device` current (switching only if needed)."""
    torch = _t()
    if device.index == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def attn_fwd_chunked(q, k, v, chunk: int, kv_len: int | None = None, causal: bool = False,
                     scale: float | None = None, out=None, stream=None):
    """Chunked/streaming forward: query windows of `chunk` rows against the first
    kv_len rows of the K/V cache (see attn_fwd_chunked in include/attn.h)."""
    torch = _t()
    B, H, S_q, S_kv, D = _check(q, k, v)
    if kv_len is None:
        kv_len = S_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    dev = q.device
    st = _call(lib.attn_fwd_chunked, dev, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
               B, H, S_q, S_kv, D, int(bool(causal)), float(scale),
               _dtype_code(q), _stream_ptr(dev, stream), int(chunk), int(kv_len))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return o


def attn_fwd_varlen(q, k, v, kv_lens, causal: bool = False, scale: float | None = None, out=None, stream=None):
    """attn_fwd with per-sequence valid key lengths: sequence b attends to its
    first kv_lens[b] K/V rows (kv_lens: int32 GPU tensor [B]; see attn_fwd_varlen
    in include/attn.h)."""
    torch = _t()
    B, H, S_q, S_kv, D = _check(q, k, v)
    if (kv_lens.dtype != torch.int32 or kv_lens.dim() != 1 or kv_lens.shape[0] != B or not kv_lens.is_contiguous()
            or kv_lens.device != q.device):
        raise ValueError("kv_lens must be a contiguous int32 tensor [B] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    dev = q.device
    st = _call(lib.attn_fwd_varlen, dev, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
               B, H, S_q, S_kv, D, int(bool(causal)), float(scale), _dtype_code(q), _stream_ptr(dev, stream),
               kv_lens.data_ptr())
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return o


def splitkv_workspace_bytes(B: int, H: int, S_q: int, n_split: int) -> int:
    n = ctypes.c_size_t()
    st = lib.attn_splitkv_workspace_bytes(B, H, S_q, n_split, ctypes.byref(n))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return n.value


def splitkv_choose(B: int, H: int, S_q: int, kv_len: int, n_cu: int) -> int:
    n = ctypes.c_int()
    st = lib.attn_splitkv_choose(B, H, S_q, kv_len, n_cu, ctypes.byref(n))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return n.value


def attn_fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, kv_len: int | None = None,
                     n_split: int = 0, out=None, workspace=None, stream=None):
    """One query window against the first kv_len K/V rows with the keys split
    over n_split workgroup ranges and merged (see attn_fwd_splitkv in
    include/attn.h).  n_split=0 asks attn_splitkv_choose for this GPU's CU
    count.  workspace: a uint8 GPU tensor of at least splitkv_workspace_bytes
    bytes (allocated here when None)."""
    torch = _t()
    B, H, S_q, S_kv, D = _check(q, k, v)
    if kv_len is None:
        kv_len = S_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = q.device
    if n_split == 0:
        n_split = splitkv_choose(B, H, S_q, kv_len, torch.cuda.get_device_properties(dev).multi_processor_count)
    need = splitkv_workspace_bytes(B, H, S_q, n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    st = _call(lib.attn_fwd_splitkv, dev, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
               B, H, S_q, S_kv, D, int(bool(causal)), float(scale), _dtype_code(q), _stream_ptr(dev, stream),
               int(kv_len), int(n_split), workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return o


def attn_fwd_splitkv_noalloc(q, k, v, out, causal: bool = False, scale: float | None = None,
                             kv_len: int | None = None, n_split: int = 0, stream=None):
    """attn_fwd_splitkv with the partial states in the library's own device
    array (see attn_fwd_splitkv_noalloc in include/attn.h): neither the library
    nor this wrapper allocates, so `out` (a contiguous tensor like q) is
    required.  n_split=0 asks attn_splitkv_choose for this GPU's CU count.
    Calls that overlap in time on one GPU must not be issued (they share the
    array)."""
    torch = _t()
    B, H, S_q, S_kv, D = _check(q, k, v)
    if kv_len is None:
        kv_len = S_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = q.device
    if n_split == 0:
        n_split = splitkv_choose(B, H, S_q, kv_len, torch.cuda.get_device_properties(dev).multi_processor_count)
    o = out
    if o is None or o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    st = _call(lib.attn_fwd_splitkv_noalloc, dev, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
               B, H, S_q, S_kv, D, int(bool(causal)), float(scale), _dtype_code(q), _stream_ptr(dev, stream),
               int(kv_len), int(n_split))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return o


def attn_qkv_proj(x, w, bias=None, out=None, stream=None):
    """Fused Q/K/V projection (see attn_qkv_proj in include/attn.h): x [B, S, d],
    w [3d, d] (rows q, then k, then v; 64 rows per head), bias [3d] or None;
    returns (q, k, v), each [B, H, S, 64] in x's dtype (bfloat16 or float16).
    out: optional tuple of three such tensors to write."""
    torch = _t()
    for name, t in (("x", x), ("w", w)) + ((("bias", bias),) if bias is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.dtype != x.dtype or t.device != x.device:
            raise ValueError(f"{name} must share x's dtype and device")
    if x.dim() != 3 or x.shape[2] % 64:
        raise ValueError(f"x must be [B, S, 64*H], got {tuple(x.shape)}")
    B, S, d = x.shape
    H = d // 64
    if tuple(w.shape) != (3 * d, d) or (bias is not None and tuple(bias.shape) != (3 * d,)):
        raise ValueError(f"w must be [{3 * d}, {d}] and bias [{3 * d}]")
    outs = tuple(torch.empty((B, H, S, 64), dtype=x.dtype, device=x.device) for _ in range(3)) if out is None else out
    for t in outs:
        if tuple(t.shape) != (B, H, S, 64) or t.dtype != x.dtype or t.device != x.device or not t.is_contiguous():
            raise ValueError("out tensors must be contiguous [B, H, S, 64] like x")
    dev = x.device
    st = _call(lib.attn_qkv_proj, dev, x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
               outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, S, H, 64, _dtype_code(x),
               _stream_ptr(dev, stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return outs


def attn_kv_append(k_cache, v_cache, k_new, v_new, kv_len: int, stream=None) -> int:
    """Write k_new, v_new [B, H, n, D] into rows [kv_len, kv_len + n) of the
    caches [B, H, S_cap, D] (see attn_kv_append in include/attn.h); returns the
    grown kv_len."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, D], got {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("caches and new rows must share a dtype")
    if not (k_cache.device == v_cache.device == k_new.device == v_new.device):
        raise ValueError("caches and new rows must be on one device")
    B, H, S_cap, D = k_cache.shape
    n = k_new.shape[2]
    if v_cache.shape != k_cache.shape or k_new.shape != (B, H, n, D) or v_new.shape != k_new.shape:
        raise ValueError(f"shape mismatch k_cache{tuple(k_cache.shape)} v_cache{tuple(v_cache.shape)} "
                         f"k_new{tuple(k_new.shape)} v_new{tuple(v_new.shape)}")
    dev = k_cache.device
    st = _call(lib.attn_kv_append, dev, k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
               B, H, S_cap, int(kv_len), n, D, _dtype_code(k_cache), _stream_ptr(dev, stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return int(kv_len) + n


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, stream=None):
    """O = softmax(Q K^T * scale [+ causal mask]) V (see attn_fwd in include/attn.h)."""
    torch = _t()
    B, H, S_q, S_kv, D = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    dev = q.device
    st = _call(lib.attn_fwd, dev, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
               B, H, S_q, S_kv, D, int(bool(causal)), float(scale),
               _dtype_code(q), _stream_ptr(dev, stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return o


# The short names of the binding: attn.fwd(q, k, v, causal=..., scale=None)
# and attn.fwd_chunked(..., chunk, kv_len) are the two entry points above.
fwd = attn_fwd
fwd_chunked = attn_fwd_chunked


def sched_rows(B: int, H: int, S_q: int, causal: bool, dtype: str, n_cu: int = 256):
    """(query rows per workgroup, key split 1 or 2) of an attn_fwd launch of
    these sizes on a device with n_cu compute units."""
    r, ks = ctypes.c_int(), ctypes.c_int()
    st = lib.attn_sched_rows(B, H, S_q, int(bool(causal)), {"f32": ATTN_F32, "f16": ATTN_F16, "bf16": ATTN_BF16}[dtype],
                             n_cu, ctypes.byref(r), ctypes.byref(ks))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return r.value, ks.value


def sched_grid(B: int, H: int, S_q: int, chunk: int, kv_len: int | None = None, causal: bool = True,
               rows: int = 128) -> int:
    g = ctypes.c_int()
    st = lib.attn_sched_grid(B, H, S_q, chunk, S_q if kv_len is None else kv_len, int(bool(causal)), rows,
                             ctypes.byref(g))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return g.value


def sched_tile(B: int, H: int, S_q: int, chunk: int, block: int, kv_len: int | None = None,
               causal: bool = True, rows: int = 128):
    h, r0, r1 = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = lib.attn_sched_tile(B, H, S_q, chunk, S_q if kv_len is None else kv_len, int(bool(causal)), rows, block,
                             ctypes.byref(h), ctypes.byref(r0), ctypes.byref(r1))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return h.value, r0.value, r1.value

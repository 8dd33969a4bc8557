"""The K/V cache append and its streaming use, through the C ABI (needs an MI355X).

The append is a copy: the HIP path must equal the oracle's slice assignment
bit for bit, on raw bit patterns (NaN payloads included).  The streaming use
-- append a window's K/V rows, then attend the window's queries to the grown
cache -- must give the single chunked call's rows exactly, from a cache whose
rows past kv_len hold NaN (they must never be read)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BITS = {"bf16": (np.int16, torch.int16, torch.bfloat16), "f16": (np.int16, torch.int16, torch.float16),
        "f32": (np.int32, torch.int32, torch.float32)}


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [  # (B, H, S_cap, kv_len, n)
    (2, 3, 300, 0, 1), (2, 3, 300, 250, 50), (1, 1, 1, 0, 1), (3, 5, 1000, 17, 300),
    (7000, 10, 4, 1, 2),          # more heads than one launch dimension holds
    (1, 2, 70000, 65000, 5000),   # a long segment per head
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_append_matches_oracle_bitwise(dtype):
    A = _lib()
    npt, tit, tdt = BITS[dtype]
    info = np.iinfo(npt)
    rng = np.random.default_rng(61)
    for B, H, S, kv, n in CASES:
        say(f"[append] {dtype} B={B} H={H} S_cap={S} kv_len={kv} n={n}")
        kc, vc = rng.integers(info.min, info.max, size=(2, B, H, S, 64), dtype=npt, endpoint=True)
        kn, vn = rng.integers(info.min, info.max, size=(2, B, H, n, 64), dtype=npt, endpoint=True)
        t = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV).view(tdt) for x in (kc, vc, kn, vn)]
        grown = A.attn_kv_append(t[0], t[1], t[2], t[3], kv)
        torch.cuda.synchronize()
        assert grown == kv + n
        rk, rv = oracle.kv_append(kc, vc, kn, vn, kv)
        assert np.array_equal(t[0].view(tit).cpu().numpy(), rk)
        assert np.array_equal(t[1].view(tit).cpu().numpy(), rv)


def test_append_rejects_past_capacity():
    A = _lib()
    kc = torch.zeros(1, 2, 10, 64, device=DEV, dtype=torch.bfloat16)
    kn = torch.zeros(1, 2, 4, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(A.AttnError):
        A.attn_kv_append(kc, kc.clone(), kn, kn.clone(), 7)


def test_streaming_append_then_windows_equal_single_call():
    """Both the single call and the windows split keys the same way (few tiles)."""
    A = _lib()
    w = W.Workload("stream2", 1, 8, 3000, 3000, 64, True, ("bf16",), seed=21)
    q, k, v = (x.to(DEV) for x in W.make_inputs(w, "bf16"))
    full = A.attn_fwd_chunked(q, k, v, chunk=512, causal=True)
    kc = torch.full_like(k, float("nan"))
    vc = torch.full_like(v, float("nan"))
    out = torch.empty_like(q)
    kv = 0
    for start in range(0, 3000, 512):
        stop = min(3000, start + 512)
        kv = A.attn_kv_append(kc, vc, k[:, :, start:stop].contiguous(), v[:, :, start:stop].contiguous(), kv)
        out[:, :, start:stop] = A.attn_fwd_chunked(q[:, :, start:stop].contiguous(), kc, vc, chunk=512, kv_len=kv,
                                                   causal=True)
    torch.cuda.synchronize()
    assert kv == 3000
    assert torch.equal(out, full)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_vs_oracle(dtype):
    """A prefill window, then single-row decode steps against the growing cache."""
    A = _lib()
    w = W.Workload("decode", 2, 4, 1520, 1520, 64, True, (dtype,), seed=22)
    q, k, v = W.make_inputs(w, dtype)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    kc = torch.full((2, 4, 2048, 64), float("nan"), device=DEV, dtype=kd.dtype)
    vc = torch.full_like(kc, float("nan"))
    kv = A.attn_kv_append(kc, vc, kd[:, :, :1500].contiguous(), vd[:, :, :1500].contiguous(), 0)
    o = A.attn_fwd_chunked(qd[:, :, :1500].contiguous(), kc, vc, chunk=1500, kv_len=kv, causal=True)
    ref = oracle.attention(q[:, :, :1500], k[:, :, :1500], v[:, :, :1500], causal=True)
    compare(o.float().cpu().numpy(), ref, dtype, "prefill")
    for step in range(1500, 1520):
        kv = A.attn_kv_append(kc, vc, kd[:, :, step:step + 1].contiguous(), vd[:, :, step:step + 1].contiguous(), kv)
        o = A.attn_fwd_chunked(qd[:, :, step:step + 1].contiguous(), kc, vc, chunk=1, kv_len=kv, causal=True)
        ref = oracle.attention(q[:, :, step:step + 1], k[:, :, :step + 1], v[:, :, :step + 1], causal=True)
        compare(o.float().cpu().numpy(), ref, dtype, f"decode step {step}")

"""Out-of-bounds writes and determinism for the entry points beyond attn_fwd
(needs an MI355X).

Each output (and the split workspace) is a view into the middle of a larger
buffer whose guard bands hold a canary bit pattern; after the call every
guard element must still hold it.  Twenty repeated calls must give the same
bits (a race in LDS or in the merge would show as a difference)."""
import sys

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 4096          # elements on each side
CANARY = 0x7A5B       # a 16-bit pattern (a NaN in fp16/bf16 would hide nothing: compared as bits)


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _guarded(shape, dtype):
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.int16, device=DEV)
    return buf, buf[GUARD:GUARD + n].view(dtype).view(shape)


def _untouched(buf, n):
    lo, hi = buf[:GUARD], buf[GUARD + n:]
    return bool((lo == CANARY).all()) and bool((hi == CANARY).all())


def _inputs(B, H, S_q, S_kv, seed):
    return (x.to(DEV) for x in W.make_inputs(W.Workload("g", B, H, S_q, S_kv, 64, False, ("bf16",), seed=seed),
                                             "bf16"))


def test_varlen_output_guard_bands():
    A = _lib()
    B, H, S_q, S_kv = 3, 2, 200, 300
    q, k, v = _inputs(B, H, S_q, S_kv, 1)
    buf, o = _guarded((B, H, S_q, 64), torch.bfloat16)
    lens = torch.tensor([300, 0, 77], dtype=torch.int32, device=DEV)
    A.attn_fwd_varlen(q, k, v, lens, causal=True, out=o)
    torch.cuda.synchronize()
    assert _untouched(buf, B * H * S_q * 64)


def test_splitkv_output_and_workspace_guard_bands():
    A = _lib()
    B, H, S_q, S_kv, ns = 2, 4, 3, 5000, 7
    q, k, v = _inputs(B, H, S_q, S_kv, 2)
    buf, o = _guarded((B, H, S_q, 64), torch.bfloat16)
    need = A.splitkv_workspace_bytes(B, H, S_q, ns)
    wbuf = torch.full((need // 2 + 2 * GUARD,), CANARY, dtype=torch.int16, device=DEV)
    ws = wbuf[GUARD:GUARD + need // 2].view(torch.uint8)
    A.attn_fwd_splitkv(q, k, v, causal=True, n_split=ns, out=o, workspace=ws)
    torch.cuda.synchronize()
    assert _untouched(buf, B * H * S_q * 64)
    assert _untouched(wbuf, need // 2)


def test_qkv_projection_guard_bands():
    A = _lib()
    B, S, H = 2, 300, 3
    d = 64 * H
    g = torch.Generator(device="cpu")
    g.manual_seed(3)
    x = torch.randn((B, S, d), generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn((3 * d, d), generator=g) / d ** 0.5).to(torch.bfloat16).to(DEV)
    outs = [_guarded((B, H, S, 64), torch.bfloat16) for _ in range(3)]
    A.attn_qkv_proj(x, w, None, out=tuple(o for _, o in outs))
    torch.cuda.synchronize()
    for buf, _ in outs:
        assert _untouched(buf, B * H * S * 64)


def test_kv_append_guard_bands():
    A = _lib()
    B, H, cap, kv, n = 2, 3, 100, 40, 30
    kbuf, kc = _guarded((B, H, cap, 64), torch.bfloat16)
    vbuf, vc = _guarded((B, H, cap, 64), torch.bfloat16)
    kn = torch.randn((B, H, n, 64), device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, H, n, 64), device=DEV).to(torch.bfloat16)
    A.attn_kv_append(kc, vc, kn, vn, kv)
    torch.cuda.synchronize()
    assert _untouched(kbuf, B * H * cap * 64) and _untouched(vbuf, B * H * cap * 64)
    # rows outside [kv, kv + n) of every head keep the canary
    kb = kc.view(torch.int16)
    assert bool((kb[:, :, :kv] == CANARY).all()) and bool((kb[:, :, kv + n:] == CANARY).all())


@pytest.mark.parametrize("entry", ["varlen", "splitkv", "qkv_proj"])
def test_repeated_calls_are_bit_identical(entry):
    A = _lib()
    q, k, v = _inputs(4, 8, 300, 3000, 4)
    lens = torch.tensor([3000, 1000, 17, 2500], dtype=torch.int32, device=DEV)
    x = torch.randn((4, 300, 512), device=DEV).to(torch.bfloat16)
    w = (torch.randn((1536, 512), device=DEV) / 512 ** 0.5).to(torch.bfloat16)

    def run():
        if entry == "varlen":
            return A.attn_fwd_varlen(q, k, v, lens, causal=False)
        if entry == "splitkv":
            return A.attn_fwd_splitkv(q, k, v, causal=True, n_split=6)
        return torch.cat([t.flatten() for t in A.attn_qkv_proj(x, w)])

    first = run().view(torch.int16).clone()
    for r in range(20):
        assert torch.equal(run().view(torch.int16), first), f"{entry}: repeat {r} differs"
    torch.cuda.synchronize()

"""The fused Q/K/V projection through the C ABI (needs an MI355X).

attn_qkv_proj against oracle.qkv_projection on seeded inputs: x ~ N(0, 1),
weights ~ N(0, 1/d) (so outputs are of order one), bias ~ N(0, 0.1^2) or none;
ragged row tiles (B*S not a multiple of 256), ragged column tiles (3d not a
multiple of 256), an odd number of 64-wide K stages, bf16 and fp16; the
32 x 1024 x 1024 layer input (the large-batch attention shape) in full; and
the projection feeding attn_fwd against the oracle's attention of the
oracle's projection rounded to the same storage type."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(B, S, H, dtype, bias, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    d = 64 * H
    x = torch.randn((B, S, d), generator=g).to(DT[dtype])
    w = (torch.randn((3 * d, d), generator=g) / d ** 0.5).to(DT[dtype])
    b = (torch.randn((3 * d,), generator=g) * 0.1).to(DT[dtype]) if bias else None
    return x, w, b


CASES = [  # B, S, H, bias
    (1, 1, 1, False),
    (2, 100, 4, True),      # 200 rows: one ragged row tile; 768 columns: three full column tiles
    (3, 70, 3, True),       # 576 columns: a ragged column tile
    (1, 513, 5, True),      # K = 320: five stages (odd); 960 columns
    (2, 300, 16, False),    # d = 1024
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_projection_matches_oracle(dtype):
    A = _lib()
    for n, (B, S, H, bias) in enumerate(CASES):
        say(f"[qkv_proj] {dtype} B={B} S={S} H={H} bias={bias}")
        x, w, b = _inputs(B, S, H, dtype, bias, seed=300 + n)
        q, k, v = A.attn_qkv_proj(x.to(DEV), w.to(DEV), b.to(DEV) if b is not None else None)
        torch.cuda.synchronize()
        ref = oracle.qkv_projection(x, w, b, H)
        for name, got, r in zip("qkv", (q, k, v), ref):
            compare(got.float().cpu().numpy(), r, dtype, f"case {n} {name}")


def test_full_layer_input():
    """B=32, S=1024, d=1024 (H=16), bf16, with bias: every output element."""
    A = _lib()
    say("[qkv_proj] full 32 x 1024 x 1024 bf16")
    x, w, b = _inputs(32, 1024, 16, "bf16", True, seed=310)
    q, k, v = A.attn_qkv_proj(x.to(DEV), w.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.qkv_projection(x, w, b, 16)
    for name, got, r in zip("qkv", (q, k, v), ref):
        compare(got.float().cpu().numpy(), r, "bf16", f"full {name}")


def test_outputs_written_in_place_and_graph_replay():
    A = _lib()
    x, w, b = (t.to(DEV) for t in _inputs(2, 300, 4, "bf16", True, seed=320))
    outs = tuple(torch.full((2, 4, 300, 64), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    eager = A.attn_qkv_proj(x, w, b)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_qkv_proj(x, w, b, out=outs)
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for got, e in zip(outs, eager):
            assert torch.equal(got.view(torch.int16), e.view(torch.int16)), f"replay {r}"


@pytest.mark.parametrize("causal", [False, True])
def test_projection_feeds_attention(causal):
    """x -> attn_qkv_proj -> attn_fwd against oracle.attention of the oracle's
    projection rounded (RNE) to bf16, as the kernels store it."""
    A = _lib()
    B, S, H = 2, 257, 4
    say(f"[qkv_proj -> attn_fwd] causal={causal}")
    x, w, b = _inputs(B, S, H, "bf16", True, seed=330)
    q, k, v = A.attn_qkv_proj(x.to(DEV), w.to(DEV), b.to(DEV))
    o = A.attn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = (torch.from_numpy(t).to(torch.bfloat16) for t in oracle.qkv_projection(x, w, b, H))
    ref = oracle.attention(rq, rk, rv, causal=causal)
    compare(o.float().cpu().numpy(), ref, "bf16", "projection then attention")

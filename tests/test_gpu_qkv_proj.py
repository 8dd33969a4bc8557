"""The fused Q/K/V projection through the C ABI (needs an MI355X).

attn_qkv_proj against oracle.qkv_projection on seeded inputs: x ~ N(0, 1),
weights ~ N(0, 1/d) (so outputs are of order one), bias ~ N(0, 0.1^2) or none;
ragged row tiles (B*S not a multiple of 256), ragged column tiles (3d not a
multiple of 256), an odd number of 64-wide K stages, bf16 and fp16; the
32 x 1024 x 1024 layer input (the large-batch attention shape) in full; and
the projection feeding attn_fwd against the oracle's attention of the
oracle's projection rounded to the same storage type.

Tolerance of the projection, element by element, from its arithmetic: the
kernel multiplies 16-bit inputs (products exact in fp32), adds the K
products and the bias in fp32 in some order, and rounds once to the storage
type.  For any order of n = K + 1 fp32 additions, each rounded to nearest or
toward zero (unit u = 2^-23, covering both), the sum differs from the exact
one by at most e = g_n * sum_k |x_k w_k| + |b| scaled alike, g_n = n u / (1 - n u)
(the classic recursive-summation bound); the final rounding adds at most
u_out * (|y| + e), u_out = 2^-8 (bf16) or 2^-11 (fp16) for round to nearest,
plus half the smallest subnormal spacing of the storage type.  The sums of
absolute products come from the oracle run on |x|, |w| and |b|."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


U_OUT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
TINY = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}


def compare_projection(got, ref, absref, K, dtype, what):
    """Assert |got - ref| <= u_out (|ref| + e) + e + tiny for every element,
    e = g_{K+1} * absref; returns the largest error / bound ratio."""
    n = K + 1
    g = n * 2.0 ** -23 / (1 - n * 2.0 ** -23)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    e = g * absref
    bound = U_OUT[dtype] * (np.abs(ref) + e) + e + TINY[dtype]
    ratio = np.abs(got - ref) / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[worst] <= 1.0, (f"{what}: element {worst} got {got[worst]} ref {ref[worst]} "
                                 f"err {abs(got[worst] - ref[worst]):.3e} > bound {bound[worst]:.3e}")
    return float(ratio.max())


def _check(outs, x, w, b, H, dtype, what):
    ref = oracle.qkv_projection(x, w, b, H)
    absref = oracle.qkv_projection(x.float().abs(), w.float().abs(), None if b is None else b.float().abs(), H)
    worst = 0.0
    for name, got, r, a in zip("qkv", outs, ref, absref):
        worst = max(worst, compare_projection(got.float().cpu().numpy(), r, a, 64 * H, dtype, f"{what} {name}"))
    say(f"  worst error / bound {worst:.3f}")


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
    (4, 256, 8, True),      # 4 row blocks x 6 column tiles: dealt to the XCDs as 2 column groups x 4 row groups
    (8, 250, 4, True),      # 8 row blocks (the last ragged) x 3 column tiles: one column group x 8 row groups
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_projection_matches_oracle(dtype):
    A = _lib()
    for n, (B, S, H, bias) in enumerate(CASES):
        say(f"[qkv_proj] {dtype} B={B} S={S} H={H} bias={bias}")
        x, w, b = _inputs(B, S, H, dtype, bias, seed=300 + n)
        q, k, v = A.attn_qkv_proj(x.to(DEV), w.to(DEV), b.to(DEV) if b is not None else None)
        torch.cuda.synchronize()
        _check((q, k, v), x, w, b, H, dtype, f"case {n}")


def test_full_layer_input():
    """B=32, S=1024, d=1024 (H=16), bf16, with bias: every output element."""
    A = _lib()
    say("[qkv_proj] full 32 x 1024 x 1024 bf16")
    x, w, b = _inputs(32, 1024, 16, "bf16", True, seed=310)
    q, k, v = A.attn_qkv_proj(x.to(DEV), w.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    _check((q, k, v), x, w, b, 16, "bf16", "full")


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

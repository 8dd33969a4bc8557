"""Seeded synthetic workloads for the attention forward pass.

This module only draws inputs: it holds no attention arithmetic, and both the
oracle checks and the HIP path consume what it returns.  Every tensor is
[B, H, S, D] row-major.  Inputs are drawn as float32 N(0, sigma^2) from a
seeded torch CPU generator (bit-reproducible on any host) and then rounded to
the storage dtype with round-to-nearest-even; the oracle sees exactly those
rounded values.

The five workloads stand in for the hackathon benchmark the pages measure on
(its 13 shapes and the 100k-token "case 14" are not reproduced; only the
dimensions the pages reveal are used: B=8, S=512, d=512 on the page
"Shape-Aware Attention", section "How we built it"; S in {128, 512, 1024, 2048}
in its arithmetic-intensity table; batch 32, d_model 1024 and ~100k tokens on
the page "GPU Kernel for a Transformer Layer", section "Challenges we faced").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S_q: int
    S_kv: int
    D: int
    causal: bool
    dtypes: tuple
    sigma: float = 1.0
    seed: int = 0
    outlier_frac: float = 0.0     # fraction of K rows per (b,h) scaled by outlier_mult
    outlier_mult: float = 8.0
    chunk: int | None = None      # query-window rows for the chunked entry point
    sample_rows: int | None = None  # rows per (b,h) checked against the oracle
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)

    def flops(self) -> float:
        """Counted work 4*B*H*S_q*S_kv*D, halved for causal."""
        f = 4.0 * self.B * self.H * self.S_q * self.S_kv * self.D
        return f / 2 if self.causal else f

    def bytes(self, dtype: str) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O written once."""
        e = torch.finfo(DTYPES[dtype]).bits // 8
        return (2 * self.S_q + 2 * self.S_kv) * self.D * e * self.B * self.H


WORKLOADS = [
    Workload("c1_single_head_f32", 1, 1, 128, 128, 64, False, ("f32",), seed=1,
             note="non-causal single head, fp32, output [1,1,128,64]"),
    Workload("c2_mha_s512", 8, 8, 512, 512, 64, False, ("f32", "f16"), seed=2,
             note="non-causal multi-head (d_model=512), fp32 and fp16 copies of the same inputs"),
    Workload("c3_causal_s2048", 4, 8, 2048, 2048, 64, True, ("bf16", "f16"), seed=3,
             note="causal, key j <= query i, bf16 and fp16 separately"),
    Workload("c4_large_batch_s1024", 32, 16, 1024, 1024, 64, False, ("bf16",), sigma=0.5, seed=4,
             outlier_frac=0.01, note="non-causal, N(0,0.5^2), 1% of K rows per head x8"),
    Workload("c5_long_causal_chunked", 16, 16, 98304, 98304, 64, True, ("bf16",), seed=5,
             chunk=4096, sample_rows=256,
             note="causal, 4096-row query windows against a K/V cache growing to 98304"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def draw_f32(shape, sigma: float, gen: torch.Generator) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32) * sigma


def outlier_rows(B: int, H: int, S: int, count: int, gen: torch.Generator) -> torch.Tensor:
    """`count` distinct key-row indices per (b,h), drawn after Q, K, V."""
    keys = torch.rand((B, H, S), generator=gen)
    return torch.argsort(keys, dim=-1)[..., :count]


def make_inputs(w: Workload, dtype: str, seed: int | None = None):
    """CPU tensors (q, k, v) in the storage dtype, for workloads small enough to
    draw on the host.  The same seed gives the same fp32 draw for every dtype,
    so the fp16 copy is the RNE rounding of the fp32 inputs."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = draw_f32((w.B, w.H, w.S_q, w.D), w.sigma, g)
    k = draw_f32((w.B, w.H, w.S_kv, w.D), w.sigma, g)
    v = draw_f32((w.B, w.H, w.S_kv, w.D), w.sigma, g)
    if w.outlier_frac > 0:
        cnt = int(round(w.outlier_frac * w.S_kv))
        idx = outlier_rows(w.B, w.H, w.S_kv, cnt, g)
        mult = torch.ones((w.B, w.H, w.S_kv), dtype=torch.float32)
        mult.scatter_(-1, idx, w.outlier_mult)
        k = k * mult.unsqueeze(-1)   # power of two: exact before or after rounding
    t = DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def make_device_inputs(w: Workload, dtype: str, device, seed: int | None = None):
    """Draw directly on the device (for the long-context workload, 3.2 GB per
    tensor in bf16): torch's device generator, seeded, N(0, sigma^2) in fp32
    then rounded.  The oracle reads the resulting device bytes back."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    t = DTYPES[dtype]
    out = []
    for S in (w.S_q, w.S_kv, w.S_kv):
        x = torch.empty((w.B, w.H, S, w.D), dtype=t, device=device)
        # fill per (b,h) so no fp32 temporary of the whole tensor is needed
        for b in range(w.B):
            y = torch.randn((w.H, S, w.D), generator=g, device=device, dtype=torch.float32)
            if w.sigma != 1.0:
                y.mul_(w.sigma)
            x[b].copy_(y)
        out.append(x)
    return tuple(out)


# Rows always included in the long-context sample: both sides of the first
# window boundaries, a late boundary and the last row.
BOUNDARY_ROWS = (0, 1, 4095, 4096, 8191, 8192, 49151, 98303)


def sample_rows(w: Workload, seed: int = 5005) -> torch.Tensor:
    """[B*H, n] sorted query-row indices per (b,h): the boundary rows that fall in
    range plus uniform draws without replacement from the rest."""
    n = w.sample_rows or 256
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    fixed = torch.tensor([r for r in BOUNDARY_ROWS if r < w.S_q], dtype=torch.int64)
    rows = []
    for _ in range(w.B * w.H):
        pool = torch.ones(w.S_q, dtype=torch.bool)
        pool[fixed] = False
        cand = torch.nonzero(pool).squeeze(1)
        pick = cand[torch.randperm(cand.numel(), generator=g)[: n - fixed.numel()]]
        rows.append(torch.sort(torch.cat([fixed, pick])).values)
    return torch.stack(rows)


def multi_seed_list(count: int = 40, base: int = 100):
    """Seeds for multi-seed sweeps (40 seeds, after the page "Shape-Aware
    Attention", section "Challenges we ran into", where one configuration
    passed on only some seeds)."""
    return list(range(base, base + count))


def varlen_lengths(B: int, S_kv: int, seed: int, low: float = 0.25, edges: bool = True) -> torch.Tensor:
    """int32 [B] per-sequence key lengths for a batch padded to S_kv keys: the
    pages give no length mix, so lengths are uniform on [ceil(low*S_kv), S_kv]
    (seeded), and with ``edges`` the first few sequences take the boundary
    lengths S_kv, 1, 0 and one past a 64-key tile (where B allows)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    lo = max(1, -(-int(low * S_kv * 1000) // 1000))
    lens = torch.randint(lo, S_kv + 1, (B,), generator=g, dtype=torch.int64)
    if edges:
        for i, L in enumerate((S_kv, 1, 0, min(S_kv, 65))):
            if i < B:
                lens[i] = L
    return lens.to(torch.int32)


# Scale at which a score is exactly q.k in log2 units for the kernels
# (|scale| * log2 e rounds to 1.0 in fp32): float32(ln 2).
LN2_F32 = float(torch.tensor(0.6931471805599453, dtype=torch.float32))


def rescale_levels(S_kv: int, D: int = 64, steady: int = 8, jump: int = 17) -> torch.Tensor:
    """[S_kv, D] float32 integer key levels for the forced-rescale inputs.

    Keys come in pairs of 64-key tiles (128 keys).  Column d walks its own
    schedule with a running level m (start 0): pair 0 holds every key at 0;
    afterwards pairs cycle, with phase d % 3, through two "steady" pairs, every
    key at m + steady, and one "jump" pair, every key at m except one per
    64-key tile (offset (5d + 3) % 64) at m + jump, after which m grows by
    jump.  Past column d's last pair, 1 + (7d) % n_pairs, every key sits at
    m - 40 (weight 2^-40, nothing).  With one-hot queries and scale LN2_F32 the
    score of a key is its level, exactly, in log2 units."""
    n_pairs = (S_kv + 127) // 128
    lev = torch.empty((S_kv, D), dtype=torch.float32)
    for d in range(D):
        m, last, off = 0.0, 1 + (7 * d) % max(1, n_pairs), (5 * d + 3) % 64
        for p in range(n_pairs):
            a, b = 128 * p, min(S_kv, 128 * p + 128)
            if p == 0:
                lev[a:b, d] = 0.0
            elif p > last:
                lev[a:b, d] = m - 40.0
            elif (p - 1 + d % 3) % 3 < 2:
                lev[a:b, d] = m + steady
            else:
                lev[a:b, d] = m
                for t0 in (a, a + 64):
                    if t0 + off < b:
                        lev[t0 + off, d] = m + jump
                m += jump
    return lev


def rescale_inputs(B: int, H: int, S_q: int, S_kv: int, seed: int, D: int = 64):
    """(q, k, v) float32 CPU tensors that force the online-softmax offset to be
    raised while the accumulator holds a large share of the row's weight:
    query row i of head (b, h) is the unit vector of column (3i + 7(bH + h) + b)
    % D, every head's keys are rescale_levels, values are N(0, 1) from the
    seed.  Every level is an integer below 256, exact in bf16, fp16 and fp32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    lev = rescale_levels(S_kv, D)
    k = lev.expand(B, H, S_kv, D).contiguous()
    q = torch.zeros((B, H, S_q, D), dtype=torch.float32)
    for b in range(B):
        for h in range(H):
            cols = (3 * torch.arange(S_q) + 7 * (b * H + h) + b) % D
            q[b, h, torch.arange(S_q), cols] = 1.0
    v = torch.randn((B, H, S_kv, D), generator=g, dtype=torch.float32)
    return q, k, v

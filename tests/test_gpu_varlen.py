"""Per-sequence key lengths (key padding) through the C ABI (needs an MI355X).

attn_fwd_varlen against the oracle's attention_varlen on the same seeded
inputs, with every K/V row at or past a sequence's length set to NaN (those
rows must never be read: one NaN reaching a tile would poison its rows).
Cases span both key-split choices (few query tiles: two wave groups per tile;
many: one), ragged tiles, empty sequences, causal rows that see no key
(length below S_q), single-row decode, lengths outside [0, S_kv] (clamped),
and a 32 x 16 x 1024 batch whose sampled sequences are checked in full.  Exact
properties: all lengths equal to L gives attn_fwd_chunked(kv_len = L) bit for
bit (same split, same per-tile arithmetic)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(B, H, S_q, S_kv, dtype, seed):
    w = W.Workload("varlen", B, H, S_q, S_kv, 64, False, (dtype,), seed=seed)
    return W.make_inputs(w, dtype)


def _pad_nan(x, lens):
    x = x.clone()
    for b, L in enumerate(lens.tolist()):
        x[b, :, max(0, min(L, x.shape[2])):] = float("nan")
    return x


def _run(A, q, k, v, lens, causal, scale=None):
    o = A.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


CASES = [
    # B, H, S_q, S_kv, causal, lengths (None: drawn)
    (4, 3, 300, 520, False, [520, 1, 0, 333]),
    (4, 3, 300, 520, True, [520, 1, 0, 333]),   # causal: rows before the first key are zero
    (3, 2, 130, 64, True, [64, 63, 40]),
    (5, 2, 200, 190, False, [-5, 1000, 190, 64, 129]),   # clamped into [0, S_kv]
    (2, 4, 1, 700, True, [700, 5]),             # one query row (decode)
    (6, 24, 520, 600, False, None),             # many query tiles: one wave group per tile
    (6, 24, 520, 600, True, None),
    (70, 1, 130, 200, True, None),              # 70 sequences of one head each, lengths from 0 to 200
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_varlen_matches_oracle(dtype):
    A = _lib()
    for n, (B, H, S_q, S_kv, causal, lens) in enumerate(CASES):
        if dtype == "f16" and B * H > 20:
            continue  # the many-tile cases run in bf16 and fp32
        lens = W.varlen_lengths(B, S_kv, seed=700 + n) if lens is None else torch.tensor(lens, dtype=torch.int32)
        say(f"[varlen] {dtype} B={B} H={H} S_q={S_q} S_kv={S_kv} causal={causal} lens={lens.tolist()[:8]}")
        q, k, v = _inputs(B, H, S_q, S_kv, dtype, seed=800 + n)
        k, v = _pad_nan(k, lens), _pad_nan(v, lens)
        got = _run(A, q, k, v, lens, causal)
        ref = oracle.attention_varlen(q, k, v, lens.numpy(), causal=causal)
        compare(got, ref, dtype, f"varlen case {n}")
        # rows that see no key are exactly zero
        empty = ref == 0.0
        assert np.all(got[empty] == 0.0), f"case {n}: a row that sees no key is not zero"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_equal_chunked_bitwise(dtype, causal):
    A = _lib()
    # L >= S_q: chunked needs it when causal.  The third shape has more than
    # two 128-row query tiles per CU (the one-group kernel at three workgroups
    # per CU), a partial last query tile and a partial cache-end tile.
    for B, H, S_q, S_kv, L in ((2, 3, 257, 400, 333), (8, 16, 512, 600, 530), (4, 16, 1100, 1300, 1250)):
        say(f"[varlen=chunked] {dtype} causal={causal} B={B} H={H} S_q={S_q} S_kv={S_kv} L={L}")
        q, k, v = (x.to(DEV) for x in _inputs(B, H, S_q, S_kv, dtype, seed=31))
        lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
        a = A.attn_fwd_varlen(q, k, v, lens, causal=causal)
        c = A.attn_fwd_chunked(q, k, v, chunk=S_q, kv_len=L, causal=causal)
        torch.cuda.synchronize()
        bits = torch.int32 if dtype == "f32" else torch.int16
        assert torch.equal(a.view(bits).cpu(), c.view(bits).cpu()), "varlen with equal lengths differs from chunked"


def test_full_batch_sampled_sequences():
    """A 32 x 16 x 1024 bf16 batch (the large-batch shape) with drawn lengths;
    eight sequences, the edge lengths among them, are checked in full."""
    A = _lib()
    B, H, S = 32, 16, 1024
    w = W.Workload("varlen_c4", B, H, S, S, 64, False, ("bf16",), sigma=0.5, seed=4)
    q, k, v = W.make_inputs(w, "bf16")
    lens = W.varlen_lengths(B, S, seed=704)
    for causal in (False, True):
        say(f"[varlen full] bf16 causal={causal} B={B} H={H} S={S}")
        got = _run(A, q, k, v, lens, causal)
        pick = [0, 1, 2, 3, 10, 17, 25, 31]
        ref = oracle.attention_varlen(q[pick], k[pick], v[pick], lens.numpy()[pick], causal=causal)
        compare(got[pick], ref, "bf16", f"varlen full causal={causal}")


def test_binding_rejects_bad_lengths_tensor():
    A = _lib()
    q = torch.zeros(2, 1, 4, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_fwd_varlen(q, q, q, torch.zeros(2, dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):
        A.attn_fwd_varlen(q, q, q, torch.zeros(3, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        A.attn_fwd_varlen(q, q, q, torch.zeros(2, dtype=torch.int32))


def test_graph_replay_reads_current_lengths():
    """The lengths are read at run time: a captured call, replayed after the
    lengths tensor is rewritten in place, follows the new lengths (each replay
    against an eager call, with eager work and synchronisation in between)."""
    A = _lib()
    B, H, S_q, S_kv = 3, 4, 200, 300
    q, k, v = (x.to(DEV) for x in _inputs(B, H, S_q, S_kv, "bf16", seed=41))
    lens = torch.tensor([300, 150, 77], dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    A.attn_fwd_varlen(q, k, v, lens, causal=True, out=out)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_fwd_varlen(q, k, v, lens, causal=True, out=out)
    for new in ([300, 150, 77], [0, 299, 200], [64, 65, 1], [300, 300, 300]):
        say(f"[varlen graph] lengths {new}")
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = A.attn_fwd_varlen(q, k, v, lens.clone(), causal=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay with lengths {new}"

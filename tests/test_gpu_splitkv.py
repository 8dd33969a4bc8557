"""Keys split across workgroups with a merge of the ranges' softmax states,
through the C ABI (needs an MI355X).

attn_fwd_splitkv against the oracle (the split changes only the summation
order, so the reference is the plain attention equation): decode-like single rows and a few
rows against long caches, causal and not, bf16/fp16/fp32, range counts from 1
to more ranges than key tiles (empty ranges), ragged tiles; one range equals
attn_fwd_chunked bit for bit; graph replays equal eager calls; one workspace
serves calls of different shapes in a row; and a decode step of the
long-context cache (16 x 16 heads x 98,304 keys, bf16, one query row) with the
automatic range count, checked on sampled heads."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT_T = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(B, H, S_q, S_kv, dtype, seed):
    return W.make_inputs(W.Workload("split", B, H, S_q, S_kv, 64, False, (dtype,), seed=seed), dtype)


CASES = [
    # B, H, S_q, S_kv, kv_len, causal, range counts
    (1, 1, 1, 5000, 5000, True, (1, 2, 7, 40, 79)),      # 79 ranges over 79 tiles; some ranges empty
    (2, 3, 1, 777, 700, False, (2, 3, 16)),
    (1, 2, 3, 4100, 4100, True, (4, 9)),                  # three rows at the end of the cache
    (1, 1, 128, 128, 128, False, (2,)),                   # the single-head 128 x 128 shape
    (2, 2, 200, 3000, 2900, True, (3, 6)),                # two query tiles, a ragged one
    (1, 4, 16, 1030, 1030, False, (5,)),
    (1, 2, 100, 6000, 5900, True, (30, 47)),              # more than three merge batches: the row-parallel merge
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_splitkv_matches_oracle(dtype):
    A = _lib()
    for n, (B, H, S_q, S_kv, kv_len, causal, splits) in enumerate(CASES):
        q, k, v = _inputs(B, H, S_q, S_kv, dtype, seed=900 + n)
        # rows past kv_len hold NaN: a range must never read them
        k[:, :, kv_len:] = float("nan")
        v[:, :, kv_len:] = float("nan")
        ref = oracle.attention(q, k, v, causal=causal, kv_len=kv_len)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        for ns in splits:
            say(f"[splitkv] {dtype} B={B} H={H} S_q={S_q} S_kv={S_kv} kv_len={kv_len} causal={causal} n_split={ns}")
            o = A.attn_fwd_splitkv(qd, kd, vd, causal=causal, kv_len=kv_len, n_split=ns)
            torch.cuda.synchronize()
            compare(o.float().cpu().numpy(), ref, dtype, f"case {n} n_split {ns}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_range_equals_chunked_bitwise(dtype):
    A = _lib()
    q, k, v = (x.to(DEV) for x in _inputs(2, 3, 70, 900, dtype, seed=17))
    a = A.attn_fwd_splitkv(q, k, v, causal=True, kv_len=850, n_split=1)
    c = A.attn_fwd_chunked(q, k, v, chunk=70, kv_len=850, causal=True)
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(a.view(bits), c.view(bits))


def test_graph_replay_and_shared_workspace():
    A = _lib()
    q, k, v = (x.to(DEV) for x in _inputs(1, 8, 2, 6000, "bf16", seed=23))
    ws = torch.empty(A.splitkv_workspace_bytes(1, 8, 2, 12), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    eager = A.attn_fwd_splitkv(q, k, v, causal=True, n_split=12, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_fwd_splitkv(q, k, v, causal=True, n_split=12, workspace=ws, out=out)
    for r in range(3):
        say(f"[splitkv graph] replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        # eager work on the same workspace in between, with another shape
        q2, k2, v2 = (x.to(DEV) for x in _inputs(1, 2, 1, 3000, "bf16", seed=24 + r))
        o2 = A.attn_fwd_splitkv(q2, k2, v2, causal=False, n_split=5, workspace=ws)
        torch.cuda.synchronize()
        compare(o2.float().cpu().numpy(), oracle.attention(q2.cpu(), k2.cpu(), v2.cpu()), "bf16", "between replays")


def test_rejects_small_workspace():
    A = _lib()
    q, k, v = (x.to(DEV) for x in _inputs(1, 2, 1, 3000, "bf16", seed=3))
    ws = torch.empty(A.splitkv_workspace_bytes(1, 2, 1, 4) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(A.AttnError):
        A.attn_fwd_splitkv(q, k, v, n_split=4, workspace=ws)


def test_decode_step_of_the_long_cache():
    """16 x 16 heads, 98,304 cached keys, one query row (bf16), automatic range
    count; 16 heads spread over the batch are checked against the oracle."""
    A = _lib()
    w = W.Workload("decode", 16, 16, 1, 98304, 64, True, ("bf16",), seed=55)
    q, k, v = W.make_device_inputs(w, "bf16", DEV)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ns = A.splitkv_choose(16, 16, 1, 98304, n_cu)
    say(f"[splitkv decode] n_split={ns}")
    o = A.attn_fwd_splitkv(q, k, v, causal=True)
    torch.cuda.synchronize()
    heads = [(b, h) for b, h in zip(range(16), (0, 5, 15, 7, 3, 11, 9, 1, 14, 2, 8, 12, 6, 10, 4, 13))]
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    qs, ks, vs = (x[bs, hs].unsqueeze(0).cpu() for x in (q, k, v))   # [1, 16, S, 64]
    ref = oracle.attention(qs, ks, vs, causal=True)
    compare(o[bs, hs].unsqueeze(0).float().cpu().numpy(), ref, "bf16", "decode step")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_loop_append_then_split_attention(dtype):
    """A decode loop on a growing cache: a 1000-row prefill, then 12 steps that
    each append one K/V row (attn_kv_append) and attend that step's query
    row to the grown cache with the automatic range count.  Every step is
    checked against the oracle on the cache as it stands; rows past kv_len
    hold NaN and must never be read."""
    A = _lib()
    B, H, cap, pre, steps = 2, 8, 1100, 1000, 12
    q_all, k_all, v_all = _inputs(B, H, pre + steps, pre + steps, dtype, seed=41)
    kc = torch.full((B, H, cap, 64), float("nan"), dtype=DT_T[dtype], device=DEV)
    vc = torch.full_like(kc, float("nan"))
    kv = A.attn_kv_append(kc, vc, k_all[:, :, :pre].contiguous().to(DEV), v_all[:, :, :pre].contiguous().to(DEV), 0)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    for t in range(steps):
        kv = A.attn_kv_append(kc, vc, k_all[:, :, kv:kv + 1].contiguous().to(DEV),
                              v_all[:, :, kv:kv + 1].contiguous().to(DEV), kv)
        q = q_all[:, :, kv - 1:kv].contiguous()
        say(f"[decode loop] {dtype} step {t} kv_len={kv} n_split={A.splitkv_choose(B, H, 1, kv, n_cu)}")
        o = A.attn_fwd_splitkv(q.to(DEV), kc, vc, causal=True, kv_len=kv)
        torch.cuda.synchronize()
        ref = oracle.attention(q, k_all[:, :, :kv], v_all[:, :, :kv], causal=True)
        compare(o.float().cpu().numpy(), ref, dtype, f"decode step {t}")

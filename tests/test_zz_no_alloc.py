"""attn_fwd_splitkv_noalloc through the C ABI (needs an MI355X): the
no-allocation variant of attn_fwd_splitkv, its partial states in the library's
own device array, gives attn_fwd_splitkv's output bit for bit -- same kernels,
same ranges -- on two calls in a row, the second smaller than the first (the
array keeps the first call's states), and both match the fp64 oracle within
the parity tolerance.  Neither the call nor its binding allocates device
memory through torch."""
import sys

import pytest
import torch

import oracle
import workloads as W
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [  # (B, H, S_q, S_kv, kv_len, causal, n_split): the second of each pair is smaller
    ((2, 4, 16, 3000, 2900, True, 5), (1, 2, 3, 1000, 1000, False, 3)),     # at most 32 rows: 32-row tiles
    ((4, 8, 1, 4096, 4096, True, 8), (1, 1, 1, 700, 650, True, 2)),
    ((1, 4, 130, 1100, 1100, True, 3), (1, 2, 40, 600, 600, False, 2)),     # 128-row tiles
    ((1, 2, 1, 8192, 8000, True, 20), (1, 1, 1, 2000, 1999, True, 9)),      # more ranges than one merge batch
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_noalloc_equals_workspace_entry_point(dtype):
    import transformer_attention_04_amd as A
    for pair_n, pair in enumerate(CASES):
        for n, (B, H, S_q, S_kv, kv_len, causal, n_split) in enumerate(pair):
            say(f"[noalloc] {dtype} case {pair_n}.{n}: B{B} H{H} S_q{S_q} S_kv{S_kv} kv_len{kv_len} "
                f"causal={causal} n_split={n_split}")
            w = W.Workload("noalloc", B, H, S_q, S_kv, 64, causal, (dtype,), seed=400 + 10 * pair_n + n)
            q, k, v = W.make_inputs(w, dtype)
            qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
            ws = torch.empty(A.splitkv_workspace_bytes(B, H, S_q, n_split), dtype=torch.uint8, device=DEV)
            ref_gpu = A.attn_fwd_splitkv(qd, kd, vd, causal=causal, kv_len=kv_len, n_split=n_split, workspace=ws)
            out = torch.full_like(qd, float("nan"))
            torch.cuda.synchronize()
            # torch's cumulative count of device allocations: the call makes none
            before = torch.cuda.memory_stats(DEV)["allocation.all.allocated"]
            got = A.attn_fwd_splitkv_noalloc(qd, kd, vd, out, causal=causal, kv_len=kv_len, n_split=n_split)
            torch.cuda.synchronize()
            assert torch.cuda.memory_stats(DEV)["allocation.all.allocated"] == before
            assert got is out
            assert torch.equal(out, ref_gpu), "differs from attn_fwd_splitkv with the same ranges"
            ref = oracle.attention(q, k, v, causal=causal, kv_len=kv_len)
            _, ratio = compare(out.float().cpu().numpy(), ref, dtype, f"noalloc {dtype} {pair_n}.{n}")
            say(f"[noalloc]   equal to attn_fwd_splitkv; worst err/bound vs oracle {ratio:.3f}")


def test_noalloc_rejects_states_beyond_the_array():
    import transformer_attention_04_amd as A
    q = torch.zeros(1, 1, 7944, 64, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, 1, 9000, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(A.AttnError) as e:
        A.attn_fwd_splitkv_noalloc(q, kv, kv, out, causal=True, n_split=8)
    assert e.value.status == A.ATTN_E_WORKSPACE

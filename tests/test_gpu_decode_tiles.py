"""Decode-sized calls at realistic batch sizes through the C ABI (needs an MI355X).

A call with at most 32 query rows per head runs 32-row tiles: one query group
per workgroup, its keys split between two waves (attn_sched_rows reports the
choice), directly through attn_fwd and inside every key range of
attn_fwd_splitkv.  Each shape is compared with the oracle element by element,
eager and after graph replays, for bf16, fp16 and fp32: one query row against
1,024 keys for 32 x 16 heads (no split), against 2,048 keys for 4 x 8 heads
(the automatic range count splits), and 16 rows against 4,096 keys (several
rows, bottom-right causal, eight ranges)."""
import sys

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


SHAPES = [  # B, H, S_q, S_kv, causal
    (32, 16, 1, 1024, True),
    (4, 8, 1, 2048, True),
    (8, 8, 16, 4096, True),
    (3, 5, 7, 999, False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_shapes_match_oracle(dtype):
    A = _lib()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    for n, (B, H, S_q, S_kv, causal) in enumerate(SHAPES):
        assert A.sched_rows(B, H, S_q, causal, dtype, n_cu) == (32, 2)
        q, k, v = W.make_inputs(W.Workload("dec", B, H, S_q, S_kv, 64, causal, (dtype,), seed=1300 + n), dtype)
        ref = oracle.attention(q, k, v, causal=causal)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        ns = A.splitkv_choose(B, H, S_q, S_kv, n_cu)
        say(f"[decode] {dtype} B{B} H{H} S_q{S_q} S_kv{S_kv} causal={causal}: {ns} range(s)")
        o_direct = A.attn_fwd(qd, kd, vd, causal=causal)
        o_split = A.attn_fwd_splitkv(qd, kd, vd, causal=causal, n_split=ns)
        torch.cuda.synchronize()
        compare(o_direct.float().cpu().numpy(), ref, dtype, f"decode direct {dtype} {B}x{H}x{S_q}x{S_kv}")
        compare(o_split.float().cpu().numpy(), ref, dtype, f"decode split {dtype} {B}x{H}x{S_q}x{S_kv}")
        # graph replays write the same bits as the eager calls
        out_d, out_s = torch.empty_like(qd), torch.empty_like(qd)
        ws = torch.empty(max(A.splitkv_workspace_bytes(B, H, S_q, ns), 16), dtype=torch.uint8, device=DEV)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            A.attn_fwd(qd, kd, vd, causal=causal, out=out_d)
            A.attn_fwd_splitkv(qd, kd, vd, causal=causal, n_split=ns, out=out_s, workspace=ws)
        for r in range(3):
            out_d.fill_(float("nan"))
            out_s.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_d, o_direct), f"direct replay {r}"
            assert torch.equal(out_s, o_split), f"split replay {r}"

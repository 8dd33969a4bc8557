"""The online-softmax rescale on the device (needs an MI355X).

Online softmax keeps a running offset m, sum l and accumulator per row and,
when a key block raises m to m', multiplies l and the accumulator by
2^(m - m') (page "GPU Kernel for a Transformer Layer", section "What we
learned").  workloads.rescale_inputs makes that happen on purpose: every row
meets blocks whose scores jump 17 log2 units above its offset after blocks
that already hold about a third of its weight, so each jump rescales a large,
non-zero state by 2^-17 (tests/test_rescale_inputs.py shows, on the CPU, that a
rescale kept at 1 or inverted then fails the tolerance).  Every kernel path
that carries the state runs on them and is compared with the fp64 oracle
element by element: one and two wave groups per query tile, the chunked
windows, keys split across workgroups with the merge, and per-sequence
lengths; bf16, fp16 and fp32; causal and not."""
import sys

import pytest
import torch

import oracle
import workloads as W
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
SCALE = W.LN2_F32


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _lib():
    import transformer_attention_04_amd as A
    return A


def _inputs(B, H, S_q, S_kv, dtype, seed):
    q, k, v = W.rescale_inputs(B, H, S_q, S_kv, seed)
    t = DT[dtype]
    return q.to(t), k.to(t), v.to(t)


GRIDS = [  # (B, H, S, what), in 128-row query tiles on 256 CUs (A.sched_rows gives the launch's choice):
    (1, 4, 1100, "two wave groups, 64-row tiles (16-bit)"),           # 36 tiles
    (4, 8, 2048, "two wave groups, 128-row tiles"),                   # 512 tiles: two per CU
    (8, 8, 1100, "one wave group"),                                   # 576 tiles
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forced_rescale_matches_oracle(dtype):
    A = _lib()
    for B, H, S, what in GRIDS:
        q, k, v = _inputs(B, H, S, S, dtype, seed=31)
        assert torch.equal(q.float(), W.rescale_inputs(B, H, S, S, 31)[0])  # exact in the storage type
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        for causal in (False, True):
            rows, ks = A.sched_rows(B, H, S, causal, dtype, torch.cuda.get_device_properties(0).multi_processor_count)
            say(f"[rescale] {dtype} {what} B{B} H{H} S{S} causal={causal}: {rows}-row tiles, key split {ks}")
            ref = oracle.attention(q, k, v, causal=causal, scale=SCALE)
            o = A.attn_fwd(qd, kd, vd, causal=causal, scale=SCALE)
            torch.cuda.synchronize()
            err, ratio = compare(o.float().cpu().numpy(), ref, dtype, f"rescale {what} causal={causal} {dtype}")
            oc = A.attn_fwd_chunked(qd, kd, vd, chunk=300, causal=causal, scale=SCALE)
            torch.cuda.synchronize()
            assert torch.equal(oc, o), "chunked windows differ from the single call"
            say(f"[rescale]   max|err| {err:.3e}, worst err/bound {ratio:.3f}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forced_rescale_split_keys(dtype):
    A = _lib()
    B, H, S_q, S_kv = 1, 4, 130, 1100
    q, k, v = _inputs(B, H, S_q, S_kv, dtype, seed=32)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        ref = oracle.attention(q, k, v, causal=causal, scale=SCALE)
        for n_split in (2, 3, 7, 12, 17):  # 12, 17: more ranges than one merge batch (8), so the merge rescales too
            o = A.attn_fwd_splitkv(qd, kd, vd, causal=causal, scale=SCALE, n_split=n_split)
            torch.cuda.synchronize()
            _, ratio = compare(o.float().cpu().numpy(), ref, dtype, f"split {n_split} causal={causal} {dtype}")
            say(f"[rescale] split {n_split} causal={causal} {dtype}: worst err/bound {ratio:.3f}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forced_rescale_per_sequence_lengths(dtype):
    A = _lib()
    B, H, S = 4, 2, 1100
    q, k, v = _inputs(B, H, S, S, dtype, seed=33)
    lens = torch.tensor([1100, 700, 333, 1050], dtype=torch.int32)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        ref = oracle.attention_varlen(q, k, v, lens.numpy(), causal=causal, scale=SCALE)
        o = A.attn_fwd_varlen(qd, kd, vd, lens.to(DEV), causal=causal, scale=SCALE)
        torch.cuda.synchronize()
        _, ratio = compare(o.float().cpu().numpy(), ref, dtype, f"varlen causal={causal} {dtype}")
        say(f"[rescale] varlen causal={causal} {dtype}: worst err/bound {ratio:.3f}")

"""Seeded random shapes over every launch shape and entry point (needs an MI355X).

attn_sched_rows picks a launch shape from B, H, S_q, causal, the dtype and the
CU count: 128-row query tiles with one wave group per tile, 128-row tiles whose
keys are split between two wave groups, 64-row and 32-row tiles with the key
split.  For each dtype this test draws shapes from a fixed generator, sorts them
by the shape the rule gives on this GPU, keeps three per (shape, causal) bucket
and runs each through one of attn_fwd, attn_fwd_chunked (random window and
cache length), attn_fwd_varlen (random per-sequence lengths, some empty or past
the cache) and attn_fwd_splitkv (random range count), comparing every element
with the oracle (attention, or attention_varlen).  The plan of cases
(launch_plan.py) is drawn on the host; test_copy_addresses.py emulates every
address of the same plan on the CPU."""
import sys

import pytest
import torch

import oracle
import workloads as W
from launch_plan import ENTRIES, plan
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_case(entry, B, H, S_q, S_kv, causal, dtype, seed, args):
    """One call through the given entry point; returns (gpu output, oracle output)."""
    A = _lib()
    w = W.Workload("shape", B, H, S_q, S_kv, 64, causal, (dtype,), seed=seed)
    q, k, v = W.make_inputs(w, dtype)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if entry == 0:
        o = A.attn_fwd(qd, kd, vd, causal=causal)
        ref = oracle.attention(q, k, v, causal=causal)
    elif entry == 1:
        o = A.attn_fwd_chunked(qd, kd, vd, chunk=args["chunk"], kv_len=args["kv_len"], causal=causal)
        ref = oracle.attention(q, k, v, causal=causal, kv_len=args["kv_len"])
    elif entry == 2:
        o = A.attn_fwd_varlen(qd, kd, vd, torch.from_numpy(args["lens"]).to(DEV), causal=causal)
        ref = oracle.attention_varlen(q, k, v, args["lens"], causal=causal)
    else:
        o = A.attn_fwd_splitkv(qd, kd, vd, causal=causal, kv_len=args["kv_len"], n_split=args["n_split"])
        ref = oracle.attention(q, k, v, causal=causal, kv_len=args["kv_len"])
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ref


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_random_shapes_every_launch_shape(dtype):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    A = _lib()
    cases = plan(dtype, n_cu)
    shapes = sorted({A.sched_rows(B, H, S_q, causal, dtype, n_cu) for _, _, B, H, S_q, _, causal, _, _ in cases})
    say(f"[shapes] {dtype} on {n_cu} CUs: launch shapes drawn {shapes}")
    want = {(128, 1), (128, 2), (64, 2), (32, 2)}
    assert want <= set(shapes), f"the draw missed launch shapes {sorted(want - set(shapes))}"
    for label, entry, B, H, S_q, S_kv, causal, seed, args in cases:
        what = f"{ENTRIES[entry]} {dict((k, v.tolist()[:6] if hasattr(v, 'tolist') else v) for k, v in args.items())}"
        say(f"[shapes] {label} {what}")
        got, ref = run_case(entry, B, H, S_q, S_kv, causal, dtype, seed, args)
        compare(got, ref, dtype, f"{label} {what}")
    say(f"[shapes] {dtype}: {len(cases)} cases match the oracle")

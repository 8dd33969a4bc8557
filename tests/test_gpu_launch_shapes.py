"""Seeded random shapes over every launch shape and entry point (needs an MI355X).

attn_sched_rows picks a launch shape from B, H, S_q, causal, the dtype and the
CU count: 128-row query tiles with one wave group per tile, 128-row tiles whose
keys are split between two wave groups, 64-row and 32-row tiles with the key
split.  For each dtype this test draws shapes from a fixed generator, sorts them
by the shape the rule gives on this GPU, keeps three per (shape, causal) bucket
and runs each through one of attn_fwd, attn_fwd_chunked (random window and
cache length), attn_fwd_varlen (random per-sequence lengths, some empty or past
the cache) and attn_fwd_splitkv (random range count), comparing every element
with the oracle (attention, or attention_varlen)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PER_BUCKET = 3
MAX_PAIRS = 6e7  # B*H*S_q*S_kv per case: the oracle stays well under a second


def _lib():
    import transformer_attention_04_amd as A
    return A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def draw_cases(dtype, n_cu, seed):
    """Buckets {(rows, key_split, causal): [(B, H, S_q, S_kv), ...]} from a
    seeded draw; shapes past MAX_PAIRS are skipped."""
    A = _lib()
    rng = np.random.RandomState(seed)
    buckets = {}
    for _ in range(20000):
        heads = int(np.exp(rng.uniform(0.0, np.log(1400.0))))
        B = int(rng.randint(1, min(heads, 24) + 1))
        H = max(1, heads // B)
        S_q = int(rng.randint(1, 33)) if rng.rand() < 0.3 else int(rng.randint(33, 420))
        causal = bool(rng.rand() < 0.5)
        S_kv = int(rng.randint(S_q if causal else 1, S_q + 400))
        if B * H * S_q * S_kv > MAX_PAIRS:
            continue
        key = A.sched_rows(B, H, S_q, causal, dtype, n_cu) + (causal,)
        b = buckets.setdefault(key, [])
        if len(b) < PER_BUCKET:
            b.append((B, H, S_q, S_kv))
    return buckets


def run_case(entry, B, H, S_q, S_kv, causal, dtype, seed, rng):
    """One call through the given entry point; returns (what, gpu output, oracle output)."""
    A = _lib()
    w = W.Workload("shape", B, H, S_q, S_kv, 64, causal, (dtype,), seed=seed)
    q, k, v = W.make_inputs(w, dtype)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lo = S_q if causal else 1
    if entry == 0:
        what = "attn_fwd"
        o = A.attn_fwd(qd, kd, vd, causal=causal)
        ref = oracle.attention(q, k, v, causal=causal)
    elif entry == 1:
        chunk = int(rng.randint(1, S_q + 1))
        kv_len = int(rng.randint(lo, S_kv + 1))
        what = f"attn_fwd_chunked chunk={chunk} kv_len={kv_len}"
        o = A.attn_fwd_chunked(qd, kd, vd, chunk=chunk, kv_len=kv_len, causal=causal)
        ref = oracle.attention(q, k, v, causal=causal, kv_len=kv_len)
    elif entry == 2:
        lens = rng.randint(0, S_kv + 4, size=B).astype(np.int32)
        what = f"attn_fwd_varlen lens={lens.tolist()[:6]}{'...' if B > 6 else ''}"
        o = A.attn_fwd_varlen(qd, kd, vd, torch.from_numpy(lens).to(DEV), causal=causal)
        ref = oracle.attention_varlen(q, k, v, lens, causal=causal)
    else:
        n_split = int(rng.randint(1, 7))
        kv_len = int(rng.randint(lo, S_kv + 1))
        what = f"attn_fwd_splitkv n_split={n_split} kv_len={kv_len}"
        o = A.attn_fwd_splitkv(qd, kd, vd, causal=causal, kv_len=kv_len, n_split=n_split)
        ref = oracle.attention(q, k, v, causal=causal, kv_len=kv_len)
    torch.cuda.synchronize()
    return what, o.float().cpu().numpy(), ref


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_random_shapes_every_launch_shape(dtype):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    seed = {"bf16": 71, "f16": 72, "f32": 73}[dtype]
    buckets = draw_cases(dtype, n_cu, seed)
    shapes = sorted({k[:2] for k in buckets})
    say(f"[shapes] {dtype} on {n_cu} CUs: launch shapes drawn {shapes}")
    want = {(128, 1), (128, 2), (64, 2), (32, 2)}
    assert want <= set(shapes), f"the draw missed launch shapes {sorted(want - set(shapes))}"
    rng = np.random.RandomState(seed + 1000)
    n = 0
    for bi, key in enumerate(sorted(buckets)):
        rows, ks, causal = key
        for ci, (B, H, S_q, S_kv) in enumerate(buckets[key]):
            entry = (bi + ci) % 4
            label = f"{dtype} rows={rows} ks={ks} B{B} H{H} S_q{S_q} S_kv{S_kv} causal={causal}"
            say(f"[shapes] {label} entry {entry}")
            what, got, ref = run_case(entry, B, H, S_q, S_kv, causal, dtype, 2000 + 97 * bi + ci, rng)
            compare(got, ref, dtype, f"{label} {what}")
            n += 1
    say(f"[shapes] {dtype}: {n} cases match the oracle")

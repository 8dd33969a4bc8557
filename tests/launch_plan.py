"""The seeded plan of random launch-shape cases (host only): drawn once, run on
the GPU by test_gpu_launch_shapes.py and emulated address by address on the
CPU by test_copy_addresses.py."""
import numpy as np

import transformer_attention_04_amd as A

PER_BUCKET = 3
MAX_PAIRS = 6e7  # B*H*S_q*S_kv per case: the oracle stays well under a second


def draw_cases(dtype, n_cu, seed):
    """Buckets {(rows, key_split, causal): [(B, H, S_q, S_kv), ...]} from a
    seeded draw; shapes past MAX_PAIRS are skipped."""
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


SEEDS = {"bf16": 71, "f16": 72, "f32": 73}
ENTRIES = ("attn_fwd", "attn_fwd_chunked", "attn_fwd_varlen", "attn_fwd_splitkv")


def plan(dtype, n_cu=256):
    """The cases of one dtype, in order: (label, entry, B, H, S_q, S_kv,
    causal, input seed, entry arguments).  Deterministic, host only."""
    seed = SEEDS[dtype]
    buckets = draw_cases(dtype, n_cu, seed)
    rng = np.random.RandomState(seed + 1000)
    cases = []
    for bi, key in enumerate(sorted(buckets)):
        rows, ks, causal = key
        for ci, (B, H, S_q, S_kv) in enumerate(buckets[key]):
            entry = (bi + ci) % 4
            lo = S_q if causal else 1
            if entry == 1:
                chunk = int(rng.randint(1, S_q + 1))
                args = dict(chunk=chunk, kv_len=int(rng.randint(lo, S_kv + 1)))
            elif entry == 2:
                args = dict(lens=rng.randint(0, S_kv + 4, size=B).astype(np.int32))
            elif entry == 3:
                # few ranges (one merge thread per row and chunk), or, for small row counts, more than 24
                # (the merge that deals each row's ranges to sixteen thread groups)
                many = B * H * S_q <= 4096 and rng.rand() < 0.5
                n_split = int(rng.randint(25, 65)) if many else int(rng.randint(1, 7))
                args = dict(n_split=n_split, kv_len=int(rng.randint(lo, S_kv + 1)))
            else:
                args = {}
            label = f"{dtype} rows={rows} ks={ks} B{B} H{H} S_q{S_q} S_kv{S_kv} causal={causal}"
            cases.append((label, entry, B, H, S_q, S_kv, causal, 2000 + 97 * bi + ci, args))
    return cases

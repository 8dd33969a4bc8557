"""The forced-rescale inputs (workloads.rescale_inputs) on the CPU: they make
the online-softmax offset rise while the accumulator already holds a large
share of a row's weight, and a mistake in that rescale shows at the parity
tolerance.

Online softmax (page "GPU Kernel for a Transformer Layer", section "What we
learned") keeps per row an offset m, a sum l and an accumulator acc over key
blocks; when a block raises m to m', l and acc are multiplied by
alpha = 2^(m - m').  `online_model` below runs that update block by block in
float64 with the two raise rules the kernels use (every block whose maximum
exceeds m by more than 8 log2 units; or only when some lane's block sum at the
old offset exceeds 2^15), so the inputs can be judged without a GPU: the model
with the right alpha matches the oracle, and the same model with alpha kept at
1, or inverted, fails the bf16 tolerance on most rows.  The GPU test of these
inputs is tests/test_gpu_rescale.py."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import TOL

BN = 64
P_LIMIT = 2.0 ** 15
LAZY = 8.0
# keys of a 32-key block held by half-wave hf: 8*(r//4) + 4*hf + r%4, r < 16
LANE_KEYS = [np.array([8 * (r // 4) + 4 * hf + r % 4 for r in range(16)]) for hf in (0, 1)]


def online_model(q, k, v, causal, rule, alpha_mode="right", kv_len=None):
    """Block-by-block online softmax of one head in log2 units (the inputs'
    scale makes a score exactly q.k in log2 units).  rule: "max" raises the
    offset whenever a block's maximum exceeds it by more than 8; "lazy" looks
    at the maximum only when the offset is unset or some lane's block sum at the
    current offset exceeds 2^15.  Returns (o, stats) with stats['raises'] the
    raises of a row that had a non-zero sum, and stats['share'] the weight the
    rows' accumulators held, after their last such raise, relative to the final
    sum."""
    S_q, S_kv = q.shape[0], k.shape[0]
    kv_len = S_kv if kv_len is None else kv_len
    s = q.astype(np.float64) @ k[:kv_len].astype(np.float64).T
    pos = np.arange(S_q)[:, None] + (kv_len - S_q)
    if causal:
        s = np.where(np.arange(kv_len)[None, :] <= pos, s, -np.inf)
    m = np.full(S_q, -np.inf)
    l = np.zeros(S_q)
    acc = np.zeros((S_q, v.shape[1]))
    raises = np.zeros(S_q, np.int64)
    share = np.zeros(S_q)
    for t0 in range(0, kv_len, BN):
        st = s[:, t0:t0 + BN]
        x = st.max(axis=1)
        with np.errstate(invalid="ignore", over="ignore"):
            if rule == "max":
                look = np.ones(S_q, bool)
            else:
                look = ~np.isfinite(m)
                mo = np.where(np.isfinite(m), m, 0.0)
                for blk in range(0, st.shape[1], 32):
                    for lk in LANE_KEYS:
                        idx = blk + lk[lk < st.shape[1] - blk]
                        look |= np.exp2(st[:, idx] - mo[:, None]).sum(axis=1) > P_LIMIT
            up = look & np.isfinite(x) & (~np.isfinite(m) | (x > m + LAZY))
            if alpha_mode == "right":
                alpha = np.exp2(m - x)
            elif alpha_mode == "one":
                alpha = np.ones(S_q)
            else:  # "inverted"
                alpha = np.exp2(x - m)
            alpha = np.where(np.isfinite(m), alpha, 0.0)
        real = up & (l > 0)
        raises += real
        l = np.where(up, l * alpha, l)
        acc = np.where(up[:, None], acc * alpha[:, None], acc)
        m = np.where(up, x, m)
        old = l.copy()
        p = np.exp2(st - np.where(np.isfinite(m), m, 0.0)[:, None])
        l = l + p.sum(axis=1)
        acc = acc + p @ v[t0:t0 + BN].astype(np.float64)
        with np.errstate(invalid="ignore", divide="ignore"):
            share = np.where(real, old / l, share)
    with np.errstate(invalid="ignore", divide="ignore"):
        # share is relative to the sum right after the raise block; rescale it
        # to the final sum below
        o = acc / l[:, None]
    return o, {"raises": raises, "share": share, "l": l}


def _head(B=1, H=2, S=1100, causal=False, seed=4321):
    q, k, v = W.rescale_inputs(B, H, S, S, seed)
    ref = oracle.attention(q, k, v, causal=causal, scale=W.LN2_F32)
    return q.numpy(), k.numpy(), v.numpy(), ref


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rule", ["max", "lazy"])
def test_right_rescale_matches_oracle_and_raises_happen(causal, rule):
    q, k, v, ref = _head(causal=causal)
    atol, rtol = TOL["bf16"]
    for h in range(q.shape[1]):
        o, st = online_model(q[0, h], k[0, h], v[0, h], causal, rule)
        # the oracle scales by float32(ln 2) = ln 2 (1 + 2.7e-9): weights at
        # levels up to ~60 differ from exact powers of two by ~2e-7 relative
        assert np.allclose(o, ref[0, h], atol=1e-6, rtol=1e-6)
        lived = st["raises"] > 0
        # most rows are raised at least once over a non-zero sum, and the
        # state carried through the last such raise is a large share of the
        # row's final weight (so a wrong alpha cannot hide)
        assert lived.mean() > (0.5 if causal else 0.8)
        assert np.median(st["share"][lived]) > 0.1
        assert np.isclose(o, ref[0, h], atol=atol, rtol=rtol).all()


@pytest.mark.parametrize("mode", ["one", "inverted"])
@pytest.mark.parametrize("rule", ["max", "lazy"])
def test_wrong_rescale_fails_the_tolerance(mode, rule):
    q, k, v, ref = _head()
    atol, rtol = TOL["bf16"]
    for h in range(q.shape[1]):
        with np.errstate(all="ignore"):
            o, _ = online_model(q[0, h], k[0, h], v[0, h], False, rule, alpha_mode=mode)
        bad = ~np.isclose(o, ref[0, h], atol=atol, rtol=rtol).all(axis=1)
        assert bad.mean() > 0.5, f"alpha {mode}: only {bad.mean():.2f} of rows fail"


def test_levels_are_exact_in_every_storage_type():
    lev = W.rescale_levels(4096)
    assert (lev == lev.round()).all() and lev.abs().max() < 256
    for t in (torch.bfloat16, torch.float16):
        assert torch.equal(lev.to(t).float(), lev)
    assert (torch.tensor(W.LN2_F32, dtype=torch.float64) * 1.4426950408889634).float().item() == 1.0

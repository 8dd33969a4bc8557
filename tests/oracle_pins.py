"""Pins for the fp64 attention oracle: checks against facts that do not come from
the oracle itself.

Every check takes ``attn`` -- a callable with the signature of
``oracle.attention`` -- and raises AssertionError on failure, so the same checks
run against the real oracle (test_oracle_pins.py) and against deliberately
broken copies of it (test_oracle_mutants.py).

Sources of truth used here, none of which is the oracle's own code:
  * closed forms of the attention equation (page "Shape-Aware Attention",
    section "Inspiration"):
    zero queries give the (prefix) mean of V; a row that sees one key returns
    that key's value row; a dominant one-hot score selects one value row; a
    two-key row is a logistic blend; adding a per-row constant to every score
    changes nothing;
  * exact invariants: value scaling by 2^k, constant values, permutations;
  * a library special case: torch's CPU float64 scaled_dot_product_attention
    with an explicit boolean mask;
  * 50-digit brute force with mpmath on tiny shapes.
"""
from __future__ import annotations

import math

import numpy as np
import torch

RNG_SEED = 20261202


def _rng(off=0):
    return np.random.default_rng(RNG_SEED + off)


def _randn(rng, shape, step=None):
    x = rng.standard_normal(shape).astype(np.float32)
    if step is not None:  # values on a grid, so sums stay exact in fp32
        x = (np.round(x / step) * step).astype(np.float32)
    return x


def _visible_mask(S_q, kv_len, causal):
    """[S_q, kv_len] bool: key j visible to query row i (bottom-right causal)."""
    i = np.arange(S_q)[:, None]
    j = np.arange(kv_len)[None, :]
    if not causal:
        return np.ones((S_q, kv_len), dtype=bool)
    return j <= (kv_len - S_q + i)


# --------------------------------------------------------------------------
# library special case
# --------------------------------------------------------------------------
def sdpa_reference(q, k, v, causal, scale, kv_len=None):
    """torch CPU float64 SDPA with an explicit boolean mask (bottom-right)."""
    S_q = q.shape[2]
    kv_len = k.shape[2] if kv_len is None else kv_len
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k[:, :, :kv_len], dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v[:, :, :kv_len], dtype=np.float64))
    mask = torch.from_numpy(_visible_mask(S_q, kv_len, causal))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.numpy()


SDPA_SHAPES = [
    # B, H, S_q, S_kv, D, causal, kv_len, scale
    (1, 1, 1, 1, 1, False, None, None),
    (1, 1, 7, 7, 3, True, None, None),
    (2, 3, 5, 9, 8, False, None, None),
    (2, 3, 5, 9, 8, True, None, None),
    (1, 2, 9, 9, 16, True, None, 0.37),
    (1, 2, 4, 12, 64, True, 10, None),     # query window at the end of a partly filled cache
    (2, 1, 6, 12, 64, False, 7, None),
    (1, 1, 33, 65, 64, True, None, -0.2),  # negative scale
    (3, 2, 17, 17, 5, False, None, 2.5),
]


def check_sdpa(attn):
    for n, (B, H, S_q, S_kv, D, causal, kv_len, scale) in enumerate(SDPA_SHAPES):
        r = _rng(n)
        q = _randn(r, (B, H, S_q, D))
        k = _randn(r, (B, H, S_kv, D))
        v = _randn(r, (B, H, S_kv, D))
        sc = 1.0 / math.sqrt(D) if scale is None else scale
        got = attn(q, k, v, causal=causal, scale=sc, kv_len=kv_len)
        ref = sdpa_reference(q, k, v, causal, sc, kv_len)
        err = np.max(np.abs(got - ref))
        assert np.all(np.isfinite(got)), f"non-finite output, shape {n}"
        assert err <= 1e-12, f"SDPA shape {n}: max err {err}"


# --------------------------------------------------------------------------
# brute force at 50 digits
# --------------------------------------------------------------------------
def _mp_attention(q, k, v, causal, scale, kv_len):
    import mpmath
    mpmath.mp.dps = 50
    B, H, S_q, D = q.shape
    out = np.zeros((B, H, S_q, D))
    for b in range(B):
        for h in range(H):
            for i in range(S_q):
                p = kv_len - S_q + i
                js = range(p + 1) if causal else range(kv_len)
                s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[b, h, i, d])) * mpmath.mpf(float(k[b, h, j, d]))
                                                     for d in range(D)) for j in js]
                w = [mpmath.e ** x for x in s]  # no max shift needed at 50 digits for these magnitudes
                tot = mpmath.fsum(w)
                for d in range(D):
                    out[b, h, i, d] = float(mpmath.fsum(wj * mpmath.mpf(float(v[b, h, j, d])) for wj, j in zip(w, js)) / tot)
    return out


def check_bruteforce(attn, cases=200):
    """200 random tiny cases (S_q <= S_kv <= 8, D <= 4, both masks, partly
    filled caches, scales of either sign) against a 50-digit evaluation."""
    r = _rng(1000)
    for n in range(cases):
        B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
        S_kv = int(r.integers(1, 9))
        S_q = int(r.integers(1, S_kv + 1))
        D = int(r.integers(1, 5))
        causal = bool(r.integers(0, 2))
        kv_len = int(r.integers(S_q if causal else 1, S_kv + 1))
        scale = float(r.uniform(-1.5, 1.5))
        q = _randn(r, (B, H, S_q, D)); k = _randn(r, (B, H, S_kv, D)); v = _randn(r, (B, H, S_kv, D))
        got = attn(q, k, v, causal=causal, scale=scale, kv_len=kv_len)
        ref = _mp_attention(q, k, v, causal, scale, kv_len)
        err = np.max(np.abs(got - ref))
        assert err <= 1e-14, f"brute-force case {n} {(B, H, S_q, S_kv, D, causal, kv_len)}: err {err}"


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def check_zero_queries(attn):
    """Q = 0: every visible score is 0, so each row is the plain mean of the
    visible value rows (all of them, or the causal prefix 0..p_i)."""
    r = _rng(2000)
    B, H, S_q, S_kv, D = 2, 2, 6, 11, 8
    q = np.zeros((B, H, S_q, D), np.float32)
    k = _randn(r, (B, H, S_kv, D)); v = _randn(r, (B, H, S_kv, D))
    for causal in (False, True):
        for kv_len in (S_kv, 8):
            got = attn(q, k, v, causal=causal, scale=0.125, kv_len=kv_len)
            for i in range(S_q):
                n = (kv_len - S_q + i + 1) if causal else kv_len
                ref = v[:, :, :n, :].astype(np.float64).mean(axis=2)
                assert np.max(np.abs(got[:, :, i] - ref)) <= 1e-14, f"Q=0 causal={causal} row {i}"


def check_causal_first_row(attn):
    """Causal with S_q = S_kv: row 0 sees only key 0, so o_0 = v_0 exactly."""
    r = _rng(2100)
    q = _randn(r, (2, 3, 9, 16)); k = _randn(r, (2, 3, 9, 16)); v = _randn(r, (2, 3, 9, 16))
    got = attn(q, k, v, causal=True, scale=0.25)
    assert np.array_equal(got[:, :, 0], v[:, :, 0].astype(np.float64)), "causal row 0 != V[0]"


def check_single_key(attn):
    """S_kv = 1 (or kv_len = 1): every row returns value row 0 exactly."""
    r = _rng(2200)
    q = _randn(r, (1, 2, 5, 8)); k = _randn(r, (1, 2, 4, 8)); v = _randn(r, (1, 2, 4, 8))
    got = attn(q, k, v, causal=False, scale=0.5, kv_len=1)
    assert np.array_equal(got, np.broadcast_to(v[:, :, :1].astype(np.float64), got.shape))


def one_hot_inputs(S_q, S_kv, D, causal, seed=0, c=1024.0):
    """Keys t_r = c*e_r for r < D at distinct positions, other keys 0; query i is
    e_{r(i)} with t_{r(i)} visible to it.  With scale 1/8 the matching score is
    c/8 = 128 and every other score is 0, so the other weights are e^-128 and
    row i equals value row t_{r(i)} to far below fp64 resolution."""
    r = np.random.default_rng(seed)
    k = np.zeros((1, 1, S_kv, D), np.float32)
    pos = r.choice(S_kv, size=min(D, S_kv), replace=False)
    for rr, t in enumerate(pos):
        k[0, 0, t, rr] = c
    q = np.zeros((1, 1, S_q, D), np.float32)
    target = np.zeros(S_q, np.int64)
    for i in range(S_q):
        p = S_kv - S_q + i
        ok = [rr for rr, t in enumerate(pos) if (t <= p or not causal)]
        rr = ok[r.integers(0, len(ok))] if ok else None
        if rr is None:  # no special key visible yet: leave q_i = 0 (mean row)
            target[i] = -1
            continue
        q[0, 0, i, rr] = 1.0
        target[i] = pos[rr]
    v = r.standard_normal((1, 1, S_kv, D)).astype(np.float32)
    return q, k, v, target


def check_one_hot(attn):
    for causal in (False, True):
        q, k, v, target = one_hot_inputs(40, 96, 8, causal, seed=int(causal))
        got = attn(q, k, v, causal=causal, scale=0.125)
        for i, t in enumerate(target):
            if t >= 0:
                assert np.array_equal(got[0, 0, i], v[0, 0, t].astype(np.float64)), f"one-hot row {i} causal={causal}"


def check_two_keys(attn):
    """Two visible keys: o = sigma(s0-s1) v0 + sigma(s1-s0) v1 (logistic form)."""
    from scipy.special import expit
    r = _rng(2300)
    q = _randn(r, (1, 1, 4, 5)); k = _randn(r, (1, 1, 2, 5)); v = _randn(r, (1, 1, 2, 5))
    sc = 0.7
    got = attn(q, k, v, causal=False, scale=sc)
    qd, kd, vd = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    for i in range(4):
        s0 = sc * float(np.dot(qd[0, 0, i], kd[0, 0, 0]))
        s1 = sc * float(np.dot(qd[0, 0, i], kd[0, 0, 1]))
        ref = expit(s0 - s1) * vd[0, 0, 0] + expit(s1 - s0) * vd[0, 0, 1]
        assert np.max(np.abs(got[0, 0, i] - ref)) <= 1e-14, f"two-key row {i}"


def check_hand_examples(attn):
    """Worked by hand.  D = 1, q = 1, scale = ln 2, keys 0, 1, 2 give scores
    0, ln2, 2 ln2, so the weights are 1 : 2 : 4.
      values (7, 14, 0):  non-causal row -> (7 + 28 + 0)/7 = 5
      causal, S_q = 3:    row 0 -> 7;  row 1 -> (7 + 28)/3 = 35/3;  row 2 -> 5
    With D = 2, q = (1, -1), keys (0,0), (1,0), (0,-1) the scores are 0, ln2,
    ln2 (weights 1 : 2 : 2); values ((5, 1), (0, 2), (10, 3)) give
    ((5 + 0 + 20)/5, (1 + 4 + 6)/5) = (5, 2.2)."""
    ln2 = math.log(2.0)
    q = np.ones((1, 1, 3, 1), np.float32)
    k = np.array([0, 1, 2], np.float32).reshape(1, 1, 3, 1)
    v = np.array([7, 14, 0], np.float32).reshape(1, 1, 3, 1)
    got = attn(q, k, v, causal=False, scale=ln2)
    assert np.allclose(got[0, 0, :, 0], [5, 5, 5], rtol=0, atol=1e-13), got
    got = attn(q, k, v, causal=True, scale=ln2)
    assert np.allclose(got[0, 0, :, 0], [7, 35 / 3, 5], rtol=0, atol=1e-13), got
    q2 = np.array([1, -1], np.float32).reshape(1, 1, 1, 2)
    k2 = np.array([[0, 0], [1, 0], [0, -1]], np.float32).reshape(1, 1, 3, 2)
    v2 = np.array([[5, 1], [0, 2], [10, 3]], np.float32).reshape(1, 1, 3, 2)
    got = attn(q2, k2, v2, causal=False, scale=ln2)
    assert np.allclose(got[0, 0, 0], [5, 2.2], rtol=0, atol=1e-13), got


def check_shift_invariance(attn):
    """K -> K + 1 w^T adds q_i . w to every score of row i; O is unchanged.  The
    shift is large (|scale * q.w| up to ~1e3), beyond exp's range, so a softmax
    without its max subtraction overflows or underflows here.  Values sit on a
    1/8 grid so K + w is exact in fp32."""
    r = _rng(2400)
    B, H, S_q, S_kv, D = 1, 2, 7, 13, 8
    q = _randn(r, (B, H, S_q, D), step=0.125)
    k = _randn(r, (B, H, S_kv, D), step=0.125)
    v = _randn(r, (B, H, S_kv, D))
    w = np.full((D,), 512.0, np.float32)
    for causal in (False, True):
        a = attn(q, k, v, causal=causal, scale=0.5)
        b = attn(q, (k + w).astype(np.float32), v, causal=causal, scale=0.5)
        assert np.all(np.isfinite(b)), "shifted scores produced non-finite output"
        assert np.max(np.abs(a - b)) <= 1e-9, f"shift changed output, causal={causal}"


def check_large_score_range(attn):
    """Scores spanning more than exp's range inside one row (|s| up to ~1300):
    only a softmax that shifts by the row maximum stays finite here; compared
    with the float64 SDPA special case."""
    r = _rng(2450)
    B, H, S_q, S_kv, D = 1, 1, 4, 24, 4
    q = np.zeros((B, H, S_q, D), np.float32)
    q[..., 0] = 64.0
    q[..., 1] = _randn(r, (B, H, S_q))
    k = _randn(r, (B, H, S_kv, D))
    # key 0 gets the lowest score, so a softmax shifted by anything but the row
    # maximum (for instance by the first score) overflows
    k[..., 0] = np.linspace(-20, 20, S_kv, dtype=np.float32)[np.concatenate([[0], 1 + r.permutation(S_kv - 1)])]
    v = _randn(r, (B, H, S_kv, D))
    for causal in (False, True):
        got = attn(q, k, v, causal=causal, scale=1.0)
        ref = sdpa_reference(q, k, v, causal, 1.0)
        assert np.all(np.isfinite(got)), "large score range produced non-finite output"
        assert np.max(np.abs(got - ref)) <= 1e-12


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def check_constant_values(attn):
    r = _rng(2500)
    q = _randn(r, (2, 2, 6, 8)); k = _randn(r, (2, 2, 9, 8))
    v = np.ones((2, 2, 9, 8), np.float32)
    for causal in (False, True):
        got = attn(q, k, v, causal=causal, scale=0.3)
        assert np.max(np.abs(got - 1.0)) <= 1e-15


def check_value_scaling(attn):
    r = _rng(2600)
    q = _randn(r, (1, 2, 6, 8)); k = _randn(r, (1, 2, 9, 8)); v = _randn(r, (1, 2, 9, 8))
    for causal in (False, True):
        a = attn(q, k, v, causal=causal, scale=0.3)
        b = attn(q, k, (v * 8).astype(np.float32), causal=causal, scale=0.3)
        assert np.array_equal(b, a * 8), "O(8V) != 8 O(V)"


def check_permutations(attn):
    r = _rng(2700)
    q = _randn(r, (2, 2, 7, 8)); k = _randn(r, (2, 2, 11, 8)); v = _randn(r, (2, 2, 11, 8))
    a = attn(q, k, v, causal=False, scale=0.4)
    pk = r.permutation(11)
    b = attn(q, k[:, :, pk], v[:, :, pk], causal=False, scale=0.4)
    assert np.max(np.abs(a - b)) <= 1e-13, "joint key/value permutation changed O"
    pq = r.permutation(7)
    c = attn(q[:, :, pq], k, v, causal=False, scale=0.4)
    assert np.array_equal(c, a[:, :, pq]), "query permutation did not permute O rows"


def check_row_subset(attn):
    r = _rng(2800)
    q = _randn(r, (2, 3, 12, 8)); k = _randn(r, (2, 3, 15, 8)); v = _randn(r, (2, 3, 15, 8))
    rows = [11, 0, 5, 6]
    for causal in (False, True):
        full = attn(q, k, v, causal=causal, scale=0.3, kv_len=14)
        sub = attn(q, k, v, causal=causal, scale=0.3, kv_len=14, rows=rows)
        assert np.array_equal(sub, full[:, :, rows]), "row subset differs from full rows"


def check_causal_prefix(attn):
    """Causal row i equals the non-causal attention of the single query row i
    over the key prefix 0..p_i."""
    r = _rng(2900)
    S_q, S_kv, D = 5, 9, 8
    q = _randn(r, (1, 2, S_q, D)); k = _randn(r, (1, 2, S_kv, D)); v = _randn(r, (1, 2, S_kv, D))
    full = attn(q, k, v, causal=True, scale=0.3)
    for i in range(S_q):
        p = S_kv - S_q + i
        one = attn(q[:, :, i:i + 1], k, v, causal=False, scale=0.3, kv_len=p + 1)
        assert np.array_equal(one[:, :, 0], full[:, :, i]), f"causal prefix row {i}"


ALL_CHECKS = [
    check_sdpa, check_bruteforce, check_zero_queries, check_causal_first_row,
    check_single_key, check_one_hot, check_two_keys, check_hand_examples,
    check_shift_invariance, check_large_score_range, check_constant_values, check_value_scaling,
    check_permutations, check_row_subset, check_causal_prefix,
]


# --------------------------------------------------------------------------
# per-sequence key lengths (key padding): checks take ``attn_varlen``, a
# callable with the signature of ``oracle.attention_varlen``
# --------------------------------------------------------------------------
def sdpa_varlen_reference(q, k, v, kv_lens, causal, scale):
    """torch CPU float64 SDPA with one boolean mask per sequence, built from
    the rule itself: key j is visible to row i of sequence b iff j < L_b and,
    when causal, j <= L_b - S_q + i (L_b clamped into [0, S_kv]).  SDPA leaves
    a row with no visible key undefined (NaN); such rows are set to zero, the
    empty weighted sum."""
    B, H, S_q, _ = q.shape
    S_kv = k.shape[2]
    mask = np.zeros((B, 1, S_q, S_kv), dtype=bool)
    i = np.arange(S_q)[:, None]
    j = np.arange(S_kv)[None, :]
    for b in range(B):
        L = min(max(int(kv_lens[b]), 0), S_kv)
        vis = j < L
        if causal:
            vis = vis & (j <= L - S_q + i)
        mask[b, 0] = vis
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask),
                                                           scale=scale).numpy()
    empty = ~mask.any(axis=3, keepdims=True)  # [B,1,S_q,1]
    return np.where(np.broadcast_to(empty, out.shape), 0.0, out)


VARLEN_SHAPES = [
    # B, H, S_q, S_kv, D, causal, kv_lens, scale
    (3, 2, 5, 9, 8, False, [9, 4, 1], None),
    (3, 2, 5, 9, 8, True, [9, 5, 7], None),
    (4, 1, 6, 10, 16, True, [3, 0, 10, 6], None),   # causal rows before the first key; an empty sequence
    (2, 3, 7, 7, 64, False, [0, 7], -0.4),
    (2, 2, 33, 70, 64, True, [70, 20], 0.3),
    (5, 1, 4, 6, 3, False, [-2, 8, 6, 2, 1], 1.7),  # lengths outside [0, S_kv] are clamped
]


def _varlen_inputs(n, B, H, S_q, S_kv, D):
    r = _rng(500 + n)
    return _randn(r, (B, H, S_q, D)), _randn(r, (B, H, S_kv, D)), _randn(r, (B, H, S_kv, D))


def check_varlen_sdpa(attn_varlen):
    for n, (B, H, S_q, S_kv, D, causal, lens, scale) in enumerate(VARLEN_SHAPES):
        q, k, v = _varlen_inputs(n, B, H, S_q, S_kv, D)
        sc = 1.0 / math.sqrt(D) if scale is None else scale
        got = attn_varlen(q, k, v, lens, causal=causal, scale=sc)
        ref = sdpa_varlen_reference(q, k, v, lens, causal, sc)
        assert got.shape == ref.shape, f"varlen shape {n}: {got.shape} vs {ref.shape}"
        assert np.all(np.isfinite(got)), f"varlen shape {n}: non-finite output"
        err = np.max(np.abs(got - ref))
        assert err <= 1e-12, f"varlen SDPA shape {n}: max err {err}"


def check_varlen_padding_ignored(attn_varlen):
    # Rows at or past a sequence's length never enter its result: NaN there
    # changes nothing.
    for n, (B, H, S_q, S_kv, D, causal, lens, scale) in enumerate(VARLEN_SHAPES):
        q, k, v = _varlen_inputs(n, B, H, S_q, S_kv, D)
        kp, vp = k.copy(), v.copy()
        for b in range(B):
            L = min(max(lens[b], 0), S_kv)
            kp[b, :, L:] = np.nan
            vp[b, :, L:] = np.nan
        a = attn_varlen(q, k, v, lens, causal=causal, scale=scale)
        c = attn_varlen(q, kp, vp, lens, causal=causal, scale=scale)
        assert np.array_equal(a, c), f"varlen shape {n}: padding rows change the result"


def check_varlen_empty_and_single_key_rows(attn_varlen):
    # L = 0: every row is zero.  Causal with L < S_q: rows i < S_q - L see no
    # key (zero); row S_q - L sees key 0 alone and returns V[0] exactly.
    B, H, S_q, S_kv, D = 3, 2, 8, 12, 5
    q, k, v = _varlen_inputs(99, B, H, S_q, S_kv, D)
    lens = [0, 3, 12]
    o = attn_varlen(q, k, v, lens, causal=True, scale=0.8)
    assert np.all(o[0] == 0.0), "an empty sequence must give zeros"
    assert np.all(o[1, :, :S_q - 3] == 0.0), "causal rows before the first key must be zero"
    assert np.array_equal(o[1, :, S_q - 3], v[1, :, 0].astype(np.float64)), "a row that sees one key returns its value"
    assert np.all(o[1, :, S_q - 3 + 1:] != 0.0)
    o = attn_varlen(q, k, v, lens, causal=False, scale=0.8)
    assert np.all(o[0] == 0.0)
    assert np.all(np.any(o[1] != 0.0, axis=-1)), "non-causal rows of a non-empty sequence see every key"


def check_varlen_full_lengths_equal_attention(attn_varlen):
    # All lengths at capacity: the padded batch is the plain batch (compared
    # with the directly masked library result, not with the oracle).
    B, H, S_q, S_kv, D = 2, 2, 6, 9, 8
    q, k, v = _varlen_inputs(77, B, H, S_q, S_kv, D)
    for causal in (False, True):
        got = attn_varlen(q, k, v, [S_kv] * B, causal=causal, scale=0.5)
        ref = sdpa_reference(q, k, v, causal, 0.5)
        assert np.max(np.abs(got - ref)) <= 1e-12


def check_varlen_batch_permutation(attn_varlen):
    # Reordering the sequences (with their lengths) reorders the results.
    B, H, S_q, S_kv, D = 4, 2, 5, 8, 4
    q, k, v = _varlen_inputs(55, B, H, S_q, S_kv, D)
    lens = np.array([8, 2, 5, 0])
    perm = np.array([2, 0, 3, 1])
    for causal in (False, True):
        a = attn_varlen(q, k, v, lens, causal=causal, scale=0.9)
        c = attn_varlen(q[perm], k[perm], v[perm], lens[perm], causal=causal, scale=0.9)
        assert np.array_equal(a[perm], c), "batch permutation"


VARLEN_CHECKS = [
    check_varlen_sdpa, check_varlen_padding_ignored, check_varlen_empty_and_single_key_rows,
    check_varlen_full_lengths_equal_attention, check_varlen_batch_permutation,
]


# --------------------------------------------------------------------------
# fused Q/K/V projection: checks take ``proj``, a callable with the signature
# of ``oracle.qkv_projection``
# --------------------------------------------------------------------------
def check_proj_bruteforce(proj):
    # explicit loops over every output element, with the stacking and head
    # split written out index by index
    r = _rng(700)
    for B, S, H, with_bias in ((1, 3, 1, True), (2, 2, 2, False), (2, 5, 1, True)):
        d = 64 * H
        x = _randn(r, (B, S, d))
        w = _randn(r, (3 * d, d))
        bias = _randn(r, (3 * d,)) if with_bias else None
        q, k, v = proj(x, w, bias, H)
        outs = (q, k, v)
        for j in range(3):
            for b in range(B):
                for h in range(H):
                    for s in range(S):
                        for e in range(64):
                            o = j * d + h * 64 + e
                            ref = math.fsum(float(x[b, s, i]) * float(w[o, i]) for i in range(d))
                            if bias is not None:
                                ref += float(bias[o])
                            assert abs(outs[j][b, h, s, e] - ref) <= 1e-9 * (1 + abs(ref)), (j, b, h, s, e)


def check_proj_identity_weights(proj):
    # W = [I; 2I; -I]: Q is the input split into heads, K twice it, V minus it
    B, S, H = 2, 7, 3
    d = 64 * H
    x = _randn(_rng(701), (B, S, d))
    eye = np.eye(d, dtype=np.float32)
    q, k, v = proj(x, np.concatenate([eye, 2 * eye, -eye]), None, H)
    heads = x.reshape(B, S, H, 64).transpose(0, 2, 1, 3).astype(np.float64)
    assert np.array_equal(q, heads) and np.array_equal(k, 2 * heads) and np.array_equal(v, -heads)


def check_proj_zero_input_gives_bias(proj):
    B, S, H = 1, 4, 2
    d = 64 * H
    bias = _randn(_rng(702), (3 * d,))
    q, k, v = proj(np.zeros((B, S, d), np.float32), _randn(_rng(703), (3 * d, d)), bias, H)
    for j, t in enumerate((q, k, v)):
        for h in range(H):
            assert np.all(t[:, h] == bias[j * d + 64 * h: j * d + 64 * h + 64].astype(np.float64))


def check_proj_head_permutation(proj):
    # permuting the heads' row blocks of each third of W permutes the output heads
    B, S, H = 2, 3, 4
    d = 64 * H
    r = _rng(704)
    x, w = _randn(r, (B, S, d)), _randn(r, (3 * d, d))
    perm = np.array([2, 0, 3, 1])
    rows = np.concatenate([j * d + 64 * p + np.arange(64) for j in range(3) for p in perm])
    a = proj(x, w, None, H)
    c = proj(x, w[rows], None, H)
    for j in range(3):
        assert np.array_equal(c[j], a[j][:, perm])


def check_proj_linearity(proj):
    B, S, H = 2, 3, 1
    d = 64 * H
    r = _rng(705)
    # inputs on a 2^-6 grid so that 0.5 x1 + 2 x2 is exact in fp32
    x1, x2 = _randn(r, (B, S, d), step=2.0 ** -6), _randn(r, (B, S, d), step=2.0 ** -6)
    w, bias = _randn(r, (3 * d, d)), _randn(r, (3 * d,))
    f = lambda x: proj(x, w, bias, H)
    a, b2, c = f(x1), f(x2), f((0.5 * x1 + 2.0 * x2).astype(np.float32))
    z = f(np.zeros_like(x1))
    for j in range(3):
        lhs = c[j] - z[j]
        rhs = 0.5 * (a[j] - z[j]) + 2.0 * (b2[j] - z[j])
        assert np.max(np.abs(lhs - rhs)) <= 1e-9


PROJ_CHECKS = [check_proj_bruteforce, check_proj_identity_weights, check_proj_zero_input_gives_bias,
               check_proj_head_permutation, check_proj_linearity]

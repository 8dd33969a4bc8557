"""The oracle against its pins (CPU only).

Each check in oracle_pins.py compares the oracle with something that is not the
oracle: closed forms of the attention equation, exact invariants, torch's float64 SDPA with an
explicit mask, and 50-digit brute force.  The workload-sized checks below run
the same library special case on the shapes of the five workloads (full
tensors for the small ones, a few heads of the larger ones)."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads as W


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle.attention)


@pytest.mark.parametrize("check", pins.VARLEN_CHECKS, ids=lambda f: f.__name__)
def test_varlen_pin(check):
    check(oracle.attention_varlen)


@pytest.mark.parametrize("check", pins.PROJ_CHECKS, ids=lambda f: f.__name__)
def test_projection_pin(check):
    check(oracle.qkv_projection)


def _heads(x, n):
    return x[:1, :n].contiguous()


@pytest.mark.parametrize("name,dtype,heads", [
    ("c1_single_head_f32", "f32", None),
    ("c2_mha_s512", "f32", None),
    ("c2_mha_s512", "f16", 4),
    ("c3_causal_s2048", "bf16", 2),
    ("c4_large_batch_s1024", "bf16", 2),
])
def test_workload_shapes_vs_sdpa(name, dtype, heads):
    w = W.BY_NAME[name]
    q, k, v = W.make_inputs(w, dtype)
    if heads:
        q, k, v = _heads(q, heads), _heads(k, heads), _heads(v, heads)
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    got = oracle.attention(qf, kf, vf, causal=w.causal, scale=w.scale)
    ref = pins.sdpa_reference(qf, kf, vf, w.causal, w.scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_long_context_sampled_rows_vs_sdpa():
    """The sampled-row mode on a long causal head (shorter than the 98,304-row
    workload, same structure: boundary rows plus seeded draws) against SDPA on
    just those rows, with the bottom-right mask."""
    w = W.Workload("long_probe", 1, 2, 12288, 12288, 64, True, ("bf16",), seed=55,
                   chunk=4096, sample_rows=24)
    q, k, v = W.make_inputs(w, "bf16")
    rows = W.sample_rows(w)
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    for bh in range(2):
        r = rows[bh].numpy()
        got = oracle.attention(qf[:, bh:bh + 1], kf[:, bh:bh + 1], vf[:, bh:bh + 1],
                               causal=True, scale=w.scale, rows=r)
        # SDPA on the selected rows: a query subset needs the mask rows of those positions
        import torch
        qt = torch.from_numpy(qf[:, bh:bh + 1, r].astype(np.float64))
        kt = torch.from_numpy(kf[:, bh:bh + 1].astype(np.float64))
        vt = torch.from_numpy(vf[:, bh:bh + 1].astype(np.float64))
        mask = torch.from_numpy(np.arange(w.S_kv)[None, :] <= r[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=w.scale).numpy()
        assert np.max(np.abs(got - ref)) <= 1e-12


def test_sample_rows_recipe():
    w = W.BY_NAME["c5_long_causal_chunked"]
    small = W.Workload("s", 2, 2, w.S_q, w.S_kv, 64, True, ("bf16",), sample_rows=256)
    rows = W.sample_rows(small)
    assert rows.shape == (4, 256)
    for r in rows:
        assert len(set(r.tolist())) == 256
        assert set(W.BOUNDARY_ROWS) <= set(r.tolist())
        assert int(r.min()) >= 0 and int(r.max()) < w.S_q
    assert not all(np.array_equal(rows[0], rows[i]) for i in range(1, 4))
    assert np.array_equal(W.sample_rows(small), rows)  # seeded


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 1, 4, 8), np.float32)
    k = np.zeros((1, 1, 3, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, causal=True)          # a row would see no key
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, kv_len=4)             # kv_len > S_kv
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, rows=[4])             # row out of range
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, scale=float("inf"))


def test_thread_count_does_not_change_results():
    r = np.random.default_rng(3)
    q = r.standard_normal((2, 2, 33, 16)).astype(np.float32)
    k = r.standard_normal((2, 2, 40, 16)).astype(np.float32)
    v = r.standard_normal((2, 2, 40, 16)).astype(np.float32)
    a = oracle.attention(q, k, v, causal=True, threads=1)
    b = oracle.attention(q, k, v, causal=True, threads=4)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# the K/V cache append (a copy: pinned by brute force and its invariants)
# ---------------------------------------------------------------------------
def test_kv_append_brute_force():
    rng = np.random.default_rng(3)
    B, H, S, D, kv, n = 2, 3, 11, 5, 4, 6
    kc, vc = rng.standard_normal((2, B, H, S, D)).astype(np.float32)
    kn, vn = rng.standard_normal((2, B, H, n, D)).astype(np.float32)
    kc0, vc0 = kc.copy(), vc.copy()
    ko, vo = oracle.kv_append(kc, vc, kn, vn, kv)
    for b in range(B):
        for h in range(H):
            for r in range(S):
                for d in range(D):
                    new = kv <= r < kv + n
                    assert ko[b, h, r, d] == (kn[b, h, r - kv, d] if new else kc[b, h, r, d])
                    assert vo[b, h, r, d] == (vn[b, h, r - kv, d] if new else vc[b, h, r, d])
    assert np.array_equal(kc, kc0) and np.array_equal(vc, vc0)  # inputs untouched


def test_kv_append_two_steps_equal_one():
    rng = np.random.default_rng(4)
    kc, vc = rng.standard_normal((2, 1, 2, 20, 3))
    kn, vn = rng.standard_normal((2, 1, 2, 9, 3))
    one = oracle.kv_append(kc, vc, kn, vn, 5)
    a = oracle.kv_append(kc, vc, kn[:, :, :4], vn[:, :, :4], 5)
    two = oracle.kv_append(a[0], a[1], kn[:, :, 4:], vn[:, :, 4:], 9)
    assert np.array_equal(one[0], two[0]) and np.array_equal(one[1], two[1])


def test_kv_append_copies_bit_patterns():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=(2, 1, 1, 8, 64), dtype=np.uint16)
    bits[0, 0, 0, 0, :4] = [0x7FC1, 0xFF80, 0x7F80, 0x0001]  # NaN payload, -inf, +inf, a denormal (bf16)
    new = rng.integers(0, 1 << 16, size=(2, 1, 1, 3, 64), dtype=np.uint16)
    ko, vo = oracle.kv_append(bits[0], bits[1], new[0], new[1], 5)
    assert np.array_equal(ko[:, :, 5:8], new[0]) and np.array_equal(ko[:, :, :5], bits[0][:, :, :5])
    assert np.array_equal(vo[:, :, 5:8], new[1]) and np.array_equal(vo[:, :, :5], bits[1][:, :, :5])


def test_kv_append_rejects_overflowing_capacity():
    z = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.kv_append(z, z, np.zeros((1, 1, 3, 2)), np.zeros((1, 1, 3, 2)), 2)

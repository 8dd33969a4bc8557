"""Host-side logic of the benchmark and its clock probe library (CPU only)."""
import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

CLOCK_LIB = os.path.join(ROOT, "transformer_attention_04_amd", "libattn_clock.so")


def test_split_steps_covers_exactly_k():
    for k in (1, 3, 7, 10, 999, 12500):
        for r in (1, 2, 5, 9):
            sizes = bench.split_steps(k, r)
            assert sum(sizes) == k and len(sizes) == min(k, r)
            assert max(sizes) - min(sizes) <= 1


def test_varlen_work_counts_visible_pairs():
    # brute force over (row, key) pairs on a tiny shape
    w = W.Workload("t", 3, 2, 5, 7, 64, True, ("bf16",))
    lens = [7, 3, 0]
    pairs = 0
    for L in lens:
        for i in range(5):
            pairs += sum(1 for j in range(7) if j < L and j <= L - 5 + i)
    flops, nbytes = bench.varlen_work(w, lens, "bf16")
    assert flops == 4.0 * 64 * pairs * 2
    assert nbytes == (2 * 5 * 3 + 2 * sum(lens)) * 64 * 2 * 2
    w2 = W.Workload("t", 2, 1, 4, 6, 64, False, ("f32",))
    assert bench.varlen_work(w2, [6, 10], "f32")[0] == 4.0 * 64 * (4 * 6 + 4 * 6)  # 10 clamps to 6


def test_clock_probe_library_exports_and_checks_arguments():
    lib = ctypes.CDLL(CLOCK_LIB)
    f = lib.attn_clock_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert f(None, 1, 1, None) == 1
    assert f(0x1004, 1, 1, None) == 1        # not 8-byte aligned
    assert f(0x1000, 0, 1, None) == 2
    assert f(0x1000, 4097, 1, None) == 2
    assert f(0x1000, 1, 0, None) == 2
    assert f(0x1000, 1, (1 << 24) + 1, None) == 2


def test_mfma_probe_checks_arguments_before_any_launch():
    lib = ctypes.CDLL(CLOCK_LIB)
    f = lib.attn_mfma_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert f(None, 1, 1, 2, None) == 1
    assert f(0x1002, 1, 1, 2, None) == 1     # not 4-byte aligned
    assert f(0x1000, 0, 1, 2, None) == 2
    assert f(0x1000, 65537, 1, 2, None) == 2
    assert f(0x1000, 1, 0, 2, None) == 2
    assert f(0x1000, 1, (1 << 24) + 1, 2, None) == 2
    assert f(0x1000, 1, 1, 3, None) == 2     # unknown dtype code
    assert f(0x1000, 1, 1, -1, None) == 2


def test_copy_probe_checks_arguments_before_any_launch():
    lib = ctypes.CDLL(CLOCK_LIB)
    f = lib.attn_copy_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    assert f(None, 0x2000, 16, 1, None) == 1
    assert f(0x1000, None, 16, 1, None) == 1
    assert f(0x1008, 0x9000, 16, 1, None) == 1     # not 16-byte aligned
    assert f(0x1000, 0x9000, 0, 1, None) == 2
    assert f(0x1000, 0x9000, 24, 1, None) == 2     # not a multiple of 16
    assert f(0x1000, 0x9000, 16, 0, None) == 2
    assert f(0x1000, 0x9000, 16, 65537, None) == 2
    assert f(0x1000, 0x1010, 64, 1, None) == 2     # overlapping ranges


def test_multi_gpu_request_exits_with_a_message():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_repeats_carry_the_set_index_so_every_set_is_timed():
    # 20 steps in 5 repeats over 32 rotating sets: the repeats cover global
    # steps 0..19 (not 0..3 five times), so 20 distinct sets are timed.
    for k, r, n_sets in ((20, 5, 32), (7, 5, 3), (100, 5, 64), (3, 5, 1), (12500, 5, 32)):
        sizes = bench.split_steps(k, r)
        bases = bench.repeat_bases(sizes)
        idx = [i for b, n in zip(bases, sizes) for i in range(b, b + n)]
        assert idx == list(range(k))
        touched = {i % n_sets for i in idx}
        assert len(touched) == bench.sets_timed(k, n_sets) == min(k, n_sets)


def test_default_line_is_the_long_context_workload_with_per_config():
    assert bench.HEADLINE == "c5_long_causal_chunked"
    w = W.BY_NAME[bench.HEADLINE]
    assert (w.B, w.H, w.S_q, w.S_kv, w.D, w.causal, w.chunk, w.dtypes[0]) == (16, 16, 98304, 98304, 64, True,
                                                                            4096, "bf16")
    names = {(n, d) for n, d in bench.PER_CONFIG}
    for wl in W.WORKLOADS:
        if wl.name != bench.HEADLINE:
            for d in wl.dtypes:
                assert (wl.name, d) in names

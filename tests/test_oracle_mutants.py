"""Do the pins catch plausible mistakes?  (CPU only.)

Each mutant is a copy of oracle/attn_oracle.c with one plausible slip planted in
it (a dropped term, a wrong sign, a wrong index, an operand from the wrong
tensor, a wrong causal boundary ...).  It is compiled into a temporary
directory and every pin in oracle_pins.py is run against it; the test demands
that at least one pin fails.  The real oracle is never modified."""
import functools
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = [
    ("scale_dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("causal_excludes_diagonal", "causal ? p + 1 : kv_len;", "causal ? p : kv_len;"),
    ("causal_top_left", "const int64_t p = kv_len - S_q + i;", "const int64_t p = i;"),
    ("wrong_k_column", "(double)qi[d] * (double)kj[d]", "(double)qi[d] * (double)kj[(d + 1) % D]"),
    ("no_max_subtraction", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    ("flipped_exponent", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("no_normalisation", "out[d] = acc / l;", "out[d] = acc;"),
    ("drops_last_key", "causal ? p + 1 : kv_len;", "causal ? p + 1 : kv_len - 1;"),
    ("reversed_v_column", "(double)vh[j * D + d]", "(double)vh[j * D + (D - 1 - d)]"),
    ("row_from_list_position", "q + (bh * S_q + i) * D", "q + (bh * S_q + r) * D"),
    ("wrong_head_for_k", "k + bh * S_kv * D, v + bh * S_kv * D", "k + (bh / 2) * S_kv * D, v + bh * S_kv * D"),
    ("values_from_keys", "k + bh * S_kv * D, v + bh * S_kv * D", "k + bh * S_kv * D, k + bh * S_kv * D"),
    ("max_not_taken", "if (s[j] > m) m = s[j];", "if (0) m = s[j];"),
    ("reversed_weights", "acc += s[j] * (double)vh[j * D + d];", "acc += s[n_vis - 1 - j] * (double)vh[j * D + d];"),
    ("normaliser_from_first_key", "l += s[j];", "l = s[0];"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new):
    assert source.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mutated = source.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "libm.so")
        with open(c, "w") as f:
            f.write(mutated)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", so, c, "-lm"], check=True)
        lib = oracle.load(so)
        attn = functools.partial(oracle.attention, lib=lib)
        caught = []
        for check in pins.ALL_CHECKS:
            try:
                check(attn)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(check.__name__)
                break
        assert caught, f"mutant {name} passed every pin"


# The per-sequence layer of oracle.attention_varlen (Python over the C
# function): each mutant plants one slip in a copy of its source text, which is
# executed in the oracle module's namespace; the varlen pins must catch it.
VARLEN_MUTANTS = [
    ("first_length_for_all", "int(lens[b])", "int(lens[0])"),
    ("not_clamped_low", "min(max(int(lens[b]), 0), S_kv)", "min(int(lens[b]), S_kv)"),
    ("causal_start_off_by_one", "max(0, S_q - L) if causal", "max(0, S_q - L + 1) if causal"),
    ("causal_top_left_rows", "o[b:b + 1, :, i0:] = attention(q[b:b + 1, :, i0:]",
     "o[b:b + 1, :, i0:] = attention(q[b:b + 1, :, :S_q - i0]"),
    ("whole_cache_read", "k[b:b + 1, :, :L], v[b:b + 1, :, :L]", "k[b:b + 1], v[b:b + 1]"),
    ("empty_rows_not_zero", "o = np.zeros((B, H, S_q, D), dtype=np.float64)",
     "o = np.full((B, H, S_q, D), np.nan)"),
    ("non_causal_inner_call", "causal=causal, scale=scale, threads", "causal=False, scale=scale, threads"),
]


@pytest.mark.parametrize("name,old,new", VARLEN_MUTANTS, ids=[m[0] for m in VARLEN_MUTANTS])
def test_varlen_mutant_is_caught(name, old, new):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle.attention_varlen))
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    mutant = ns["attention_varlen"]
    caught = []
    for check in pins.VARLEN_CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(check.__name__)
            break
    assert caught, f"varlen mutant {name} passed every pin"


# The Q/K/V projection (numpy in oracle/__init__.py): one planted slip per
# mutant in a copy of its source text.
PROJ_MUTANTS = [
    ("weights_not_transposed", "y = x.reshape(B * S, d) @ w.T", "y = x.reshape(B * S, d) @ w[:d].T.repeat(3, 1).T.T"),
    ("bias_dropped", "y = y + np.asarray(_f32(bias), dtype=np.float64).reshape(1, 3 * d)", "y = y"),
    ("heads_before_thirds", "y = y.reshape(B, S, 3, H, 64)", "y = y.reshape(B, S, H, 3, 64).transpose(0, 1, 3, 2, 4)"),
    ("k_and_v_swapped", "for j in range(3))", "for j in (0, 2, 1))"),
    ("sequence_and_head_axes_kept", "y[:, :, j].transpose(0, 2, 1, 3)", "y[:, :, j].reshape(B, H, S, 64)"),
]


@pytest.mark.parametrize("name,old,new", PROJ_MUTANTS, ids=[m[0] for m in PROJ_MUTANTS])
def test_projection_mutant_is_caught(name, old, new):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle.qkv_projection))
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    mutant = ns["qkv_projection"]
    caught = []
    for check in pins.PROJ_CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
            break
    assert caught, f"projection mutant {name} passed every pin"

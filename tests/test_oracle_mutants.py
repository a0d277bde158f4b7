"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of ``oracle/attn_oracle.c`` with one plausible slip
(a dropped term, a wrong sign, scale or index, a transposed layout, a wrong
tie rule).  It is built into a temporary library and the oracle pin tests are
run against it in a subprocess; every mutant has to make them fail.  The
mistakes live only in those temporary copies, on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

MUTANTS = {
    "scale_1_over_d": ("w[j] = acc / sqrt_d;", "w[j] = acc / 128.0;"),
    "exp_sign": ("w[j] = exp(w[j] - m);", "w[j] = exp(m - w[j]);"),
    "drop_first_dim": ("for (int c = 0; c < D; ++c)\n            acc += qrow[c] * kr[c];",
                       "for (int c = 1; c < D; ++c)\n            acc += qrow[c] * kr[c];"),
    "no_normalisation": ("o[c] = acc[c] / l;", "o[c] = acc[c];"),
    "reversed_weights": ("acc[c] += w[j] * vr[c];", "acc[c] += w[Sk - 1 - j] * vr[c];"),
    "bshd_as_bhsd": ("return ((b * S + s) * H + h) * D + c;", "return ((b * H + h) * S + s) * D + c;"),
    "q_head_index_swapped": ("qrow[c] = oracle_bf16_decode(jb->q[offset_of(jb->layout, jb->H, jb->Sq, jb->b, jb->h, i, c)]);",
                             "qrow[c] = oracle_bf16_decode(jb->q[offset_of(jb->layout, jb->H, jb->Sq, jb->b, (jb->h + 1) % jb->H, i, c)]);"),
    "rtne_tie_to_odd": ("fmod(f, 2.0) == 1.0", "fmod(f, 2.0) == 0.0"),
    "rtna_strict": ("if (r >= 0.5)", "if (r > 0.5)"),
    "decode_bias": ("mag = ldexp((double)(128 + f), e - 127 - 7);", "mag = ldexp((double)(128 + f), e - 126 - 7);"),
    "no_subnormal_clamp": ("if (e < -126)\n        e = -126;", ""),
    "overflow_rtz_to_inf": ("return mode == OR_RTZ ? (sign | 0x7F7F) : (sign | 0x7F80);", "return sign | 0x7F80;"),
    "causal_diagonal_excluded": ("int64_t n = i + off + 1;", "int64_t n = i + off;"),
    "causal_bottom_right_offset_sign": ("OR_MASK_CAUSAL_TOP_LEFT ? 0 : Sk - Sq;", "OR_MASK_CAUSAL_TOP_LEFT ? 0 : Sq - Sk;"),
    "causal_mask_ignored": ("return n < Sk ? n : Sk;", "return Sk;"),
    "causal_alignments_swapped": ("OR_MASK_CAUSAL_TOP_LEFT ? 0 : Sk - Sq;", "OR_MASK_CAUSAL_TOP_LEFT ? Sk - Sq : 0;"),
    "causal_empty_row_zero": ("    if (Sk == 0)\n        return 0.0;", "    if (Sk == 0)\n        return 1.0;"),
    "gqa_k_head_modulo": ("decode_head(k, layout, H_kv, Sk, b, h / group, Kd);", "decode_head(k, layout, H_kv, Sk, b, h % H_kv, Kd);"),
    "lse_drops_the_max": ("        return m + log(l);", "        return log(l);"),
    "lse_base_two": ("        return m + log(l);", "        return m + log2(l);"),
    "lse_empty_row_nan": ("    if (m == -INFINITY)\n        return -INFINITY;\n    return NAN;",
                          "    if (m == -INFINITY)\n        return NAN;\n    return NAN;"),
    "gqa_v_head_modulo": ("decode_head(v, layout, H_kv, Sk, b, h / group, Vd);", "decode_head(v, layout, H_kv, Sk, b, h % H_kv, Vd);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "attn_oracle_mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
                    str(mut), "-lm", "-o", str(lib)], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_attention.py", "tests/test_oracle_causal.py",
                        "tests/test_oracle_gqa.py", "tests/test_oracle_lse.py", "tests/test_oracle_rounding.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


# Planted mistakes in the Python side of the oracle (the variable-length
# composition): a copy of the oracle package with one edit is put first on
# the import path, the C library stays the real one, and the varlen pins run
# against it.
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PY_MUTANTS = {
    "varlen_keys_shifted": ("np.ascontiguousarray(k[k0:k1][None]),\n                               np.ascontiguousarray(v[k0:k1][None])",
                            "np.ascontiguousarray(k[k0 + 1:k1 + 1][None]),\n                               np.ascontiguousarray(v[k0 + 1:k1 + 1][None])"),
    "varlen_queries_of_next_sequence": ("q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]",
                                        "q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[min(b + 1, B - 1)], cu_k[min(b + 2, B)]"),
    "varlen_empty_keys_zero": ("o_exact = np.full((n, D), np.nan)", "o_exact = np.zeros((n, D))"),
    "varlen_row_sequence_search": ('seq = np.searchsorted(cu_q, rows[:, 0], side="right") - 1',
                                   'seq = np.searchsorted(cu_q, rows[:, 0], side="left") - 1'),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS) + ["unmutated"])
def test_python_mutant_is_caught(name, tmp_path):
    import oracle

    old, new = PY_MUTANTS.get(name, ("", ""))
    src = open(PY_SRC).read()
    assert name == "unmutated" or src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(src.replace(old, new))
    env = dict(os.environ, ORACLE_LIB=oracle.build())
    # import the mutant first: the tests then find it in sys.modules whatever
    # pytest puts on the path
    boot = ("import sys; sys.path.insert(0, sys.argv[1]); import oracle; "
            "assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__; import pytest; "
            "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', 'tests/test_oracle_varlen.py']))")
    r = subprocess.run([sys.executable, "-c", boot, str(tmp_path)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert "AssertionError: /" not in r.stderr, r.stderr[-2000:]
    if name == "unmutated":  # the harness itself: an exact copy passes
        assert r.returncode == 0, r.stdout[-2000:]
    else:
        assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"

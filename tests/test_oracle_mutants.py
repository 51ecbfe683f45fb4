"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle's C source (compiled to a temporary library, on the CPU) makes at
least one pin fail.  Each mutant runs in a child process, so a mutant that
reads out of bounds cannot take the test runner down."""
import subprocess
import sys
from pathlib import Path

import pytest

import oracle

ROOT = Path(__file__).resolve().parents[1]
PINS = Path(__file__).resolve().parent / "oracle_pins.py"

# (name, exact text in oracle_sgemm.c, replacement)
MUTANTS = [
    ("drop_last_term", "for (int64_t t = 0; t < k; ++t) {\n            const double a",
     "for (int64_t t = 0; t < k - 1; ++t) {\n            const double a"),
    ("drop_first_term", "for (int64_t t = 0; t < k; ++t) {\n            const double a",
     "for (int64_t t = 1; t < k; ++t) {\n            const double a"),
    ("wrong_sign", "acc[j] += p;", "acc[j] -= p;"),
    ("a_transposed", "jb->A[i * jb->sa_i + t * jb->sa_t]", "jb->A[t * jb->sa_i + i * jb->sa_t]"),
    ("b_transposed", "const double p = a * (double)brow[j * jb->sb_j];",
     "const double p = a * (double)jb->B[j * jb->sb_t + t * jb->sb_j];"),
    ("b_row_index_i", "const float *brow = jb->B + t * jb->sb_t;",
     "const float *brow = jb->B + i * jb->sb_t;"),
    ("alpha_ignored", "double r = use_ab ? jb->alpha * acc[j] : 0.0;",
     "double r = use_ab ? acc[j] : 0.0;"),
    ("beta_sign", "if (jb->beta != 0.0) r += jb->beta * (double)crow[j];",
     "if (jb->beta != 0.0) r -= jb->beta * (double)crow[j];"),
    ("beta_zero_reads_c", "if (jb->beta != 0.0) r += jb->beta * (double)crow[j];",
     "r += jb->beta * (double)crow[j];"),
    ("alpha_zero_reads_ab", "const int use_ab = (k > 0 && jb->alpha != 0.0);",
     "const int use_ab = (k > 0);"),
    ("float_accumulator", "const double p = a * (double)brow[j * jb->sb_j];",
     "const double p = (double)(float)(a * (double)brow[j * jb->sb_j]); acc[j] = (float)acc[j];"),
    ("g_signed", "gacc[j] += fabs(p);", "gacc[j] += p;"),
    ("row_list_ignored", "const int64_t i = jb->rows ? jb->rows[s] : s;",
     "const int64_t i = s;"),
    ("points_drop_last", "for (int64_t t = 0; t < k; ++t) {\n                const double prod",
     "for (int64_t t = 0; t + 1 < k; ++t) {\n                const double prod"),
    ("points_transposed_b", "(double)B[t * sb_t + j * sb_j]", "(double)B[j * sb_t + t * sb_j]"),
    ("points_beta_sign", "if (db != 0.0) r += db * (double)C[i * ldc + j];",
     "if (db != 0.0) r -= db * (double)C[i * ldc + j];"),
    # transposed storage
    ("trans_a_ignored", "jb->sa_i = trans_a ? 1 : lda;\n        jb->sa_t = trans_a ? lda : 1;",
     "jb->sa_i = lda;\n        jb->sa_t = 1;"),
    ("trans_b_ignored", "jb->sb_t = trans_b ? 1 : ldb;\n        jb->sb_j = trans_b ? ldb : 1;",
     "jb->sb_t = ldb;\n        jb->sb_j = 1;"),
    ("trans_a_stride_m", "jb->sa_t = trans_a ? lda : 1;", "jb->sa_t = trans_a ? m : 1;"),
    ("trans_b_stride_n", "jb->sb_j = trans_b ? ldb : 1;", "jb->sb_j = trans_b ? n : 1;"),
    ("points_trans_b_ignored", "const int64_t sb_t = trans_b ? 1 : ldb, sb_j = trans_b ? ldb : 1;",
     "const int64_t sb_t = ldb, sb_j = 1;"),
    ("points_trans_a_ignored", "const int64_t sa_i = trans_a ? 1 : lda, sa_t = trans_a ? lda : 1;",
     "const int64_t sa_i = lda, sa_t = 1;"),
    ("trans_width_unchecked", "const int64_t wa = ta ? m : k, wb = tb ? k : n;",
     "const int64_t wa = k, wb = n;"),
    ("c_pad_written", "for (int64_t j = 0; j < n; ++j) {\n        double r",
     "for (int64_t j = 0; j < jb->ldc; ++j) {\n        double r"),
]


# mistakes planted in oracle_reduce.c
MUTANTS_REDUCE = [
    ("sum_drop_last", "for (int64_t i = 0; i < n; ++i)", "for (int64_t i = 0; i + 1 < n; ++i)"),
    ("sum_drop_first", "for (int64_t i = 0; i < n; ++i)", "for (int64_t i = 1; i < n; ++i)"),
    ("sum_float_acc", "        s += v;", "        s = (float)(s + v);"),
    ("sum_abs_signed", "a += fabs(v);", "a += v;"),
    ("sum_sign", "        s += v;", "        s -= v;"),
]


def _run_pins_on(tmp_path, sgemm_src, reduce_src):
    lib = oracle.build(sgemm_src, tmp_path / "liboracle_mutant.so", reduce_src)
    return subprocess.run([sys.executable, str(PINS), str(lib)], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name,old,new", MUTANTS_REDUCE, ids=[m[0] for m in MUTANTS_REDUCE])
def test_reduce_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.SRC_REDUCE.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mutated = tmp_path / "oracle_reduce_mutant.c"
    mutated.write_text(src.replace(old, new))
    res = _run_pins_on(tmp_path, oracle.SRC, mutated)
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.SRC.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(mutated, tmp_path / "liboracle_mutant.so")
    res = subprocess.run([sys.executable, str(PINS), str(lib)], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout}"


def test_unmutated_source_passes(tmp_path):
    lib = oracle.build(oracle.SRC, tmp_path / "liboracle_copy.so")
    res = subprocess.run([sys.executable, str(PINS), str(lib)], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr

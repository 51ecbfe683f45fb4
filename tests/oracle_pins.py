"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

No page prints output values for a concrete matrix, so the oracle is pinned
by facts that hold for the definition C_ij = sum_t A_it * B_tj (page
"GEMM优化原理", section 问题定义, eq. 1) whatever the implementation:

  * closed forms: all-ones operands give C_ij = k; A_it = 1, B_tj = t gives
    k(k-1)/2; A_it = i+1 gives k(i+1); B_tj = j+1 gives k(j+1); A_it = t,
    B_tj = t gives (k-1)k(2k-1)/6;
  * special matrices: I*B = B and A*I = A bitwise, a permutation matrix
    permutes rows exactly;
  * a library routine on a case where it is exact: integer-valued operands
    against numpy's int64 matrix product;
  * brute force: tiny random float shapes against an exact rational sum
    (fractions.Fraction), with the double-accumulation error bound
    |S - exact| <= k * 2^-53 * sum_t |A_it B_tj|;
  * invariants: transposition (B^T A^T = (AB)^T, bitwise), independence of
    the thread count, exact power-of-two scaling by alpha;
  * the alpha/beta readings: alpha = 0 leaves beta*C, beta = 0 never reads C
    (NaN there stays out), integer alpha = 1.5 / beta = 0.5 cases are exact;
  * storage: pads (NaN in A and B, a sentinel in C) are neither read nor
    written.

Each check is a function taking an ``oracle.Oracle``; it raises
AssertionError on failure.  ``tests/test_oracle.py`` runs them under pytest;
``tests/test_oracle_mutants.py`` runs this file as a script against oracle
builds with a planted mistake and expects a failure.
"""
from __future__ import annotations

import sys
from fractions import Fraction
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

import synth  # noqa: E402

NAN = np.float32(np.nan)
SENT = synth.C_SENTINEL

TAIL_SHAPES = [(1, 1, 1), (3, 5, 7), (17, 33, 31), (33, 17, 64), (31, 9, 257)]


def _pad(a: np.ndarray, ld: int, pad=NAN) -> np.ndarray:
    return synth.padded(np.asarray(a, dtype=np.float32), ld, pad)


def _run(orc, A, B, C=None, alpha=1.0, beta=0.0, m=None, n=None, k=None, **kw):
    """Call the whole-matrix oracle on padded 2-D arrays."""
    m = A.shape[0] if m is None else m
    k = k if k is not None else (A.shape[1] if B is None else B.shape[0])
    n = n if n is not None else B.shape[1]
    lda, ldb = A.shape[1], B.shape[1]
    if C is None:
        C = _pad(np.zeros((m, n), np.float32), n + 2, SENT)
    return orc.sgemm(m, n, k, alpha, A, lda, B, ldb, beta, C, C.shape[1], **kw)


def _logical(C, m, n):
    return np.asarray(C).reshape(m, -1)[:, :n]


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def pin_all_ones(orc):
    for (m, n, k) in TAIL_SHAPES + [(8, 8, 4097)]:
        A = _pad(np.ones((m, k)), k + 3)
        B = _pad(np.ones((k, n)), n + 1)
        r = _run(orc, A, B, m=m, n=n, k=k)
        got = _logical(r["C"], m, n)
        assert np.array_equal(got, np.full((m, n), k, np.float32)), (m, n, k)


def pin_arith_series(orc):
    for (m, n, k) in [(4, 6, 1), (5, 3, 100), (7, 9, 5793)]:
        t = np.arange(k, dtype=np.float32)
        A = _pad(np.ones((m, k)), k)
        B = _pad(np.repeat(t[:, None], n, axis=1), n + 5)
        got = _logical(_run(orc, A, B, m=m, n=n, k=k)["C"], m, n)
        assert np.array_equal(got, np.full((m, n), k * (k - 1) // 2, np.float32)), k


def pin_row_and_column_index(orc):
    m, n, k = 6, 5, 11
    i = np.arange(m, dtype=np.float32)
    j = np.arange(n, dtype=np.float32)
    A = _pad(np.repeat((i + 1)[:, None], k, axis=1), k + 2)
    B = _pad(np.ones((k, n)), n)
    got = _logical(_run(orc, A, B, m=m, n=n, k=k)["C"], m, n)
    assert np.array_equal(got, np.repeat((k * (i + 1))[:, None], n, axis=1)), "row"
    A = _pad(np.ones((m, k)), k)
    B = _pad(np.repeat((j + 1)[None, :], k, axis=0), n + 3)
    got = _logical(_run(orc, A, B, m=m, n=n, k=k)["C"], m, n)
    assert np.array_equal(got, np.repeat((k * (j + 1))[None, :], m, axis=0)), "col"


def pin_sum_of_squares(orc):
    m, n = 3, 4
    for k in (1, 2, 50, 300):
        t = np.arange(k, dtype=np.float32)
        A = _pad(np.repeat(t[None, :], m, axis=0), k + 1)
        B = _pad(np.repeat(t[:, None], n, axis=1), n)
        got = _logical(_run(orc, A, B, m=m, n=n, k=k)["C"], m, n)
        want = (k - 1) * k * (2 * k - 1) // 6
        assert np.array_equal(got, np.full((m, n), want, np.float32)), k


# --------------------------------------------------------------------------
# special matrices
# --------------------------------------------------------------------------
def pin_identity(orc):
    rng = np.random.default_rng(7)
    for (m, n) in [(1, 1), (5, 9), (33, 17)]:
        Bv = rng.standard_normal((m, n)).astype(np.float32)
        A = _pad(np.eye(m), m + 1)
        got = _logical(_run(orc, A, _pad(Bv, n + 2), m=m, n=n, k=m)["C"], m, n)
        assert np.array_equal(got, Bv), ("I*B", m, n)
        Av = rng.standard_normal((m, n)).astype(np.float32)
        got = _logical(_run(orc, _pad(Av, n), _pad(np.eye(n), n + 3), m=m, n=n, k=n)["C"], m, n)
        assert np.array_equal(got, Av), ("A*I", m, n)


def pin_permutation(orc):
    rng = np.random.default_rng(11)
    k, n = 13, 7
    perm = rng.permutation(k)
    P = np.zeros((k, k), np.float32)
    P[np.arange(k), perm] = 1.0
    Bv = rng.uniform(-1, 1, (k, n)).astype(np.float32)
    got = _logical(_run(orc, _pad(P, k + 2), _pad(Bv, n + 1), m=k, n=n, k=k)["C"], k, n)
    assert np.array_equal(got, Bv[perm]), "P*B"


# --------------------------------------------------------------------------
# library routine where it is exact: integer operands
# --------------------------------------------------------------------------
def pin_integer_exact(orc):
    rng = np.random.default_rng(3)
    for (m, n, k) in TAIL_SHAPES + [(40, 24, 3000)]:
        Ai = rng.integers(-3, 4, (m, k)).astype(np.int64)
        Bi = rng.integers(-3, 4, (k, n)).astype(np.int64)
        want = (Ai @ Bi).astype(np.float32)
        got = _logical(_run(orc, _pad(Ai, k + 4), _pad(Bi, n + 2), m=m, n=n, k=k)["C"], m, n)
        assert np.array_equal(got, want), (m, n, k)


# --------------------------------------------------------------------------
# brute force against exact rationals
# --------------------------------------------------------------------------
def _exact(Av, Bv, i, j):
    return sum((Fraction(float(Av[i, t])) * Fraction(float(Bv[t, j]))
                for t in range(Av.shape[1])), Fraction(0))


def pin_brute_force_fraction(orc):
    rng = np.random.default_rng(5)
    sizes = [1, 2, 3, 5, 8, 9, 17]
    for m in sizes[::2]:
        for n in sizes[1::2]:
            for k in (1, 4, 15, 33):
                Av = rng.uniform(-1, 1, (m, k)).astype(np.float32)
                Bv = rng.uniform(-1, 1, (k, n)).astype(np.float32)
                r = _run(orc, _pad(Av, k + 1), _pad(Bv, n), m=m, n=n, k=k,
                         want_s=True, want_g=True)
                C = _logical(r["C"], m, n)
                for i in range(m):
                    for j in range(n):
                        ex = _exact(Av, Bv, i, j)
                        g = r["G"][i, j]
                        s = r["S"][i, j]
                        assert abs(Fraction(s) - ex) <= Fraction(k) * Fraction(2) ** -53 * Fraction(g), (m, n, k, i, j)
                        exf = np.float32(float(ex))
                        # one rounding of (nearly) the exact value: within one ulp
                        assert abs(float(C[i, j]) - float(exf)) <= float(np.spacing(np.abs(exf))) + 1e-45, (i, j)
                        gx = sum(abs(Fraction(float(Av[i, t])) * Fraction(float(Bv[t, j]))) for t in range(k))
                        assert Fraction(g) == gx or abs(Fraction(g) - gx) <= Fraction(k) * Fraction(2) ** -53 * gx


def pin_numpy_float64(orc):
    rng = np.random.default_rng(9)
    m, n, k = 31, 33, 129
    Av = rng.standard_normal((m, k)).astype(np.float32)
    Bv = rng.standard_normal((k, n)).astype(np.float32)
    r = _run(orc, _pad(Av, k), _pad(Bv, n + 7), m=m, n=n, k=k, want_s=True, want_g=True)
    ref = Av.astype(np.float64) @ Bv.astype(np.float64)
    assert np.all(np.abs(r["S"] - ref) <= 1e-12 * r["G"]), "S vs float64 matmul"
    gref = np.abs(Av.astype(np.float64)) @ np.abs(Bv.astype(np.float64))
    assert np.allclose(r["G"], gref, rtol=1e-12, atol=0), "G vs |A||B|"


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def pin_transpose(orc):
    rng = np.random.default_rng(13)
    m, n, k = 19, 23, 41
    Av = rng.standard_normal((m, k)).astype(np.float32)
    Bv = rng.standard_normal((k, n)).astype(np.float32)
    C1 = _logical(_run(orc, _pad(Av, k), _pad(Bv, n), m=m, n=n, k=k)["C"], m, n)
    C2 = _logical(_run(orc, _pad(Bv.T.copy(), k + 1), _pad(Av.T.copy(), m + 2),
                       m=n, n=m, k=k)["C"], n, m)
    assert np.array_equal(C1, C2.T), "(AB)^T != B^T A^T"


def pin_thread_count(orc):
    rng = np.random.default_rng(17)
    m, n, k = 37, 29, 301
    A = _pad(rng.standard_normal((m, k)).astype(np.float32), k)
    B = _pad(rng.standard_normal((k, n)).astype(np.float32), n)
    base = _run(orc, A, B, m=m, n=n, k=k, threads=1)["C"]
    for t in (2, 3, 8, 64):
        assert np.array_equal(_run(orc, A, B, m=m, n=n, k=k, threads=t)["C"], base), t


def pin_alpha_power_of_two(orc):
    rng = np.random.default_rng(19)
    m, n, k = 9, 14, 65
    A = _pad(rng.standard_normal((m, k)).astype(np.float32), k)
    B = _pad(rng.standard_normal((k, n)).astype(np.float32), n)
    base = _logical(_run(orc, A, B, m=m, n=n, k=k)["C"], m, n)
    for p in (-3, 1, 7):
        got = _logical(_run(orc, A, B, alpha=2.0 ** p, m=m, n=n, k=k)["C"], m, n)
        assert np.array_equal(got, base * np.float32(2.0 ** p)), p
    got = _logical(_run(orc, A, B, alpha=-1.0, m=m, n=n, k=k)["C"], m, n)
    assert np.array_equal(got, -base), "alpha=-1"


# --------------------------------------------------------------------------
# alpha / beta readings
# --------------------------------------------------------------------------
def pin_alpha_beta_integers(orc):
    rng = np.random.default_rng(23)
    for (m, n, k) in [(5, 7, 9), (33, 17, 500)]:
        Ai = rng.integers(-3, 4, (m, k)).astype(np.int64)
        Bi = rng.integers(-3, 4, (k, n)).astype(np.int64)
        Ci = rng.integers(-3, 4, (m, n)).astype(np.int64)
        C = _pad(Ci, n + 1, SENT)
        r = _run(orc, _pad(Ai, k), _pad(Bi, n), C=C, alpha=1.5, beta=0.5, m=m, n=n, k=k)
        want = ((3 * (Ai @ Bi) + Ci) / 2.0).astype(np.float32)  # exact halves
        assert np.array_equal(_logical(r["C"], m, n), want), ("1.5/0.5", m, n, k)
        r = _run(orc, _pad(Ai, k), _pad(Bi, n), C=C, alpha=-1.0, beta=1.0, m=m, n=n, k=k)
        assert np.array_equal(_logical(r["C"], m, n), (Ci - Ai @ Bi).astype(np.float32)), "C - AB"
        r = _run(orc, _pad(Ai, k), _pad(Bi, n), C=C, alpha=1.0, beta=-2.0, m=m, n=n, k=k)
        assert np.array_equal(_logical(r["C"], m, n), (Ai @ Bi - 2 * Ci).astype(np.float32)), "AB - 2C"


def pin_alpha_zero_and_k_zero(orc):
    rng = np.random.default_rng(29)
    m, n, k = 6, 10, 8
    Cv = rng.standard_normal((m, n)).astype(np.float32)
    C = _pad(Cv, n + 2, SENT)
    A = _pad(np.full((m, k), np.nan, np.float32), k)  # never read
    B = _pad(np.full((k, n), np.inf, np.float32), n)  # never read
    got = _logical(_run(orc, A, B, C=C, alpha=0.0, beta=0.75, m=m, n=n, k=k)["C"], m, n)
    assert np.array_equal(got, (np.float64(0.75) * Cv).astype(np.float32)), "alpha=0"
    got = _logical(_run(orc, A, B, C=C, alpha=1.0, beta=-1.25, m=m, n=n, k=0)["C"], m, n)
    assert np.array_equal(got, (np.float64(-1.25) * Cv).astype(np.float32)), "k=0"
    got = _logical(_run(orc, A, B, C=C, alpha=0.0, beta=0.0, m=m, n=n, k=k)["C"], m, n)
    assert np.array_equal(got, np.zeros((m, n), np.float32)), "alpha=beta=0"


def pin_beta_zero_ignores_c(orc):
    m, n, k = 4, 6, 5
    C = _pad(np.full((m, n), np.nan, np.float32), n + 1, SENT)
    A = _pad(np.ones((m, k)), k)
    B = _pad(np.ones((k, n)), n)
    got = _logical(_run(orc, A, B, C=C, alpha=2.0, beta=0.0, m=m, n=n, k=k)["C"], m, n)
    assert np.array_equal(got, np.full((m, n), 2 * k, np.float32)), "beta=0 read C"


# --------------------------------------------------------------------------
# storage: pads, row subsets, single entries
# --------------------------------------------------------------------------
def pin_pads_untouched(orc):
    rng = np.random.default_rng(31)
    m, n, k = 21, 13, 37
    A = _pad(rng.uniform(-1, 1, (m, k)).astype(np.float32), k + 5)
    B = _pad(rng.uniform(-1, 1, (k, n)).astype(np.float32), n + 3)
    C = _pad(rng.uniform(-1, 1, (m, n)).astype(np.float32), n + 7, SENT)
    out = _run(orc, A, B, C=C, alpha=1.0, beta=1.0, m=m, n=n, k=k)["C"].reshape(m, -1)
    assert np.all(np.isfinite(out[:, :n])), "NaN pad leaked"
    assert np.array_equal(out[:, n:], C[:, n:]), "pad of C written"


def pin_rows_subset(orc):
    rng = np.random.default_rng(37)
    m, n, k = 40, 9, 77
    Ai = rng.integers(-3, 4, (m, k)).astype(np.int64)
    Bi = rng.integers(-3, 4, (k, n)).astype(np.int64)
    C = _pad(np.zeros((m, n), np.float32), n, SENT)
    rows = [0, 3, 17, 39]
    r = orc.sgemm(m, n, k, 1.0, _pad(Ai, k), k, _pad(Bi, n), n, 0.0, C, n,
                  rows=rows, want_s=True)
    out = r["C"].reshape(m, n)
    want = (Ai @ Bi).astype(np.float64)
    assert np.array_equal(out[rows], want[rows].astype(np.float32)), "listed rows"
    others = [i for i in range(m) if i not in rows]
    assert np.array_equal(out[others], np.zeros((len(others), n), np.float32)), "other rows written"
    assert np.array_equal(r["S"], want[rows]), "S of listed rows"


def pin_points(orc):
    rng = np.random.default_rng(41)
    m, n, k = 30, 26, 333
    Ai = rng.integers(-3, 4, (m, k)).astype(np.int64)
    Bi = rng.integers(-3, 4, (k, n)).astype(np.int64)
    Ci = rng.integers(-3, 4, (m, n)).astype(np.int64)
    A, B, C = _pad(Ai, k + 1), _pad(Bi, n + 2), _pad(Ci, n + 3, SENT)
    ii = np.array([0, 29, 5, 17, 29], np.int64)
    jj = np.array([0, 25, 25, 3, 0], np.int64)
    r = orc.points(m, n, k, 1.5, A, k + 1, B, n + 2, 0.5, C, n + 3, ii, jj)
    want = ((3 * (Ai @ Bi) + Ci) / 2.0)[ii, jj].astype(np.float32)
    assert np.array_equal(r["C"], want), "points int"
    Av = rng.standard_normal((m, k)).astype(np.float32)
    Bv = rng.standard_normal((k, n)).astype(np.float32)
    full = _run(orc, _pad(Av, k), _pad(Bv, n), m=m, n=n, k=k, want_s=True)
    p = orc.points(m, n, k, 1.0, _pad(Av, k), k, _pad(Bv, n), n, 0.0, None, n, ii, jj)
    ref = Av.astype(np.float64) @ Bv.astype(np.float64)
    assert np.all(np.abs(p["S"] - ref[ii, jj]) <= 1e-12 * p["G"]), "points S"
    assert np.array_equal(p["S"], full["S"][ii, jj]), "points vs rows: same ascending sum"


# --------------------------------------------------------------------------
# operands stored transposed (trans_a: A is k x m; trans_b: B is n x k)
# --------------------------------------------------------------------------
def _stored(X, trans, pad_cols):
    """Storage of logical operand X: X itself or its transpose, padded."""
    S = np.ascontiguousarray(X.T) if trans else np.asarray(X)
    return _pad(S, S.shape[1] + pad_cols)


def _run_t(orc, Av, Bv, ta, tb, Cin=None, alpha=1.0, beta=0.0, **kw):
    m, k = Av.shape
    n = Bv.shape[1]
    A, B = _stored(Av, ta, 3), _stored(Bv, tb, 5)
    C = _pad(np.zeros((m, n), np.float32) if Cin is None else Cin, n + 2, SENT)
    return orc.sgemm(m, n, k, alpha, A, A.shape[1], B, B.shape[1], beta, C, n + 2,
                     trans_a=ta, trans_b=tb, **kw)


def pin_transposed_closed_form(orc):
    """A_it = i + 1 and B_tj = t give C_ij = (i + 1) k (k - 1) / 2; A_it = t and
    B_tj = j + 1 give (j + 1) k (k - 1) / 2 -- for every storage order, with
    NaN pads, so a stored operand read with the wrong strides shows."""
    m, n, k = 7, 5, 9
    i = np.arange(m, dtype=np.float32)[:, None]
    j = np.arange(n, dtype=np.float32)[None, :]
    t_row = np.arange(k, dtype=np.float32)
    tri = k * (k - 1) / 2
    for ta in (False, True):
        for tb in (False, True):
            A1 = np.repeat(i + 1, k, axis=1)
            B1 = np.repeat(t_row[:, None], n, axis=1)
            C1 = _logical(_run_t(orc, A1, B1, ta, tb)["C"], m, n)
            assert np.array_equal(C1, np.repeat((i + 1) * tri, n, axis=1)), (ta, tb, "A=i+1")
            A2 = np.repeat(t_row[None, :], m, axis=0)
            B2 = np.repeat(j + 1, k, axis=0)
            C2 = _logical(_run_t(orc, A2, B2, ta, tb)["C"], m, n)
            assert np.array_equal(C2, np.repeat((j + 1) * tri, m, axis=0)), (ta, tb, "B=j+1")


def pin_transposed_integer_exact(orc):
    """Small integers are summed exactly; numpy int64 matmul of the logical
    operands is the reference, for all four storage orders."""
    rng = np.random.default_rng(43)
    for (m, n, k) in TAIL_SHAPES + [(12, 40, 300)]:
        Ai = rng.integers(-3, 4, (m, k)).astype(np.int64)
        Bi = rng.integers(-3, 4, (k, n)).astype(np.int64)
        Ci = rng.integers(-3, 4, (m, n)).astype(np.int64)
        want = ((3 * (Ai @ Bi) + Ci) / 2.0).astype(np.float32)
        for ta in (False, True):
            for tb in (False, True):
                r = _run_t(orc, Ai.astype(np.float32), Bi.astype(np.float32), ta, tb,
                           Cin=Ci.astype(np.float32), alpha=1.5, beta=0.5)
                assert np.array_equal(_logical(r["C"], m, n), want), (m, n, k, ta, tb)
                assert np.all(r["C"].reshape(m, -1)[:, n:] == SENT), "C pads written"


def pin_transposed_points(orc):
    rng = np.random.default_rng(47)
    m, n, k = 21, 34, 77
    Ai = rng.integers(-3, 4, (m, k)).astype(np.int64)
    Bi = rng.integers(-3, 4, (k, n)).astype(np.int64)
    ii = np.array([0, 20, 7, 20, 3], np.int64)
    jj = np.array([0, 33, 33, 0, 11], np.int64)
    want = (Ai @ Bi)[ii, jj].astype(np.float32)
    for ta in (False, True):
        for tb in (False, True):
            A, B = _stored(Ai.astype(np.float32), ta, 2), _stored(Bi.astype(np.float32), tb, 1)
            r = orc.points(m, n, k, 1.0, A, A.shape[1], B, B.shape[1], 0.0, None, n, ii, jj,
                           trans_a=ta, trans_b=tb)
            assert np.array_equal(r["C"], want), (ta, tb)


def pin_transposed_leading_dims(orc):
    """Stored widths: lda >= m for A^T (may be < k), ldb >= k for B^T (may be
    < n); one less is rejected."""
    m, n, k = 3, 9, 6
    Av = np.ones((m, k), np.float32)
    Bv = np.ones((k, n), np.float32)
    At, Bt = np.ascontiguousarray(Av.T), np.ascontiguousarray(Bv.T)   # k x m, n x k
    C = np.zeros((m, n), np.float32)
    r = orc.sgemm(m, n, k, 1.0, At, m, Bt, k, 0.0, C, n, trans_a=True, trans_b=True)
    assert np.array_equal(r["C"], np.full((m, n), k, np.float32))
    for bad in [dict(lda=m - 1, ldb=k), dict(lda=m, ldb=k - 1)]:
        try:
            orc.sgemm(m, n, k, 1.0, At, bad["lda"], Bt, bad["ldb"], 0.0, C, n,
                      trans_a=True, trans_b=True)
        except ValueError:
            continue
        raise AssertionError(f"accepted {bad}")


ALL_PINS = [
    pin_all_ones, pin_arith_series, pin_row_and_column_index, pin_sum_of_squares,
    pin_identity, pin_permutation, pin_integer_exact, pin_brute_force_fraction,
    pin_numpy_float64, pin_transpose, pin_thread_count, pin_alpha_power_of_two,
    pin_alpha_beta_integers, pin_alpha_zero_and_k_zero, pin_beta_zero_ignores_c,
    pin_pads_untouched, pin_rows_subset, pin_points,
    pin_transposed_closed_form, pin_transposed_integer_exact, pin_transposed_points,
    pin_transposed_leading_dims,
]


# --------------------------------------------------------------------------
# array sum (oracle_sum)
# --------------------------------------------------------------------------
def pin_sum_arith_series(orc):
    for n in (0, 1, 2, 7, 1000, 1 << 20):
        x = np.arange(1, n + 1, dtype=np.float32)
        s, a = orc.sum(x)
        assert s == n * (n + 1) // 2 and a == s, n


def pin_sum_integers(orc):
    rng = np.random.default_rng(43)
    for n in (5, 4097, 300001):
        xi = rng.integers(-3, 4, n).astype(np.int64)
        s, a = orc.sum(xi.astype(np.float32))
        assert s == xi.sum() and a == np.abs(xi).sum(), n


def pin_sum_exact_rational(orc):
    import math
    rng = np.random.default_rng(47)
    for n in (1, 3, 64, 1001):
        x = rng.standard_normal(n).astype(np.float32) * np.float32(1e3)
        s, a = orc.sum(x)
        exact = math.fsum(float(v) for v in x)           # correctly rounded
        aexact = math.fsum(abs(float(v)) for v in x)
        assert abs(s - exact) <= n * 2.0 ** -53 * aexact + abs(exact) * 2.0 ** -53, n
        assert abs(a - aexact) <= n * 2.0 ** -53 * aexact, n


def pin_sum_cancellation(orc):
    x = np.array([1e8, 1.0, -1e8, 0.5, 3.0, -0.25], dtype=np.float32)
    s, a = orc.sum(x)
    assert s == 4.25 and a == 2e8 + 4.75


ALL_PINS += [pin_sum_arith_series, pin_sum_integers, pin_sum_exact_rational, pin_sum_cancellation]


def main(argv):
    """Run every pin against the oracle library named on the command line.
    Exit status 0 when all pass, 1 when any fails (names printed)."""
    from oracle import Oracle
    orc = Oracle(argv[1])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - a mutant may fail in any way
            failed.append(f"{pin.__name__}: {type(e).__name__}: {e}")
    for f in failed:
        print("FAIL", f)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))

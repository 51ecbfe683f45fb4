"""Comparison of GPU results with the CPU oracle.

Floating-point bar (elementwise, C_in the input C, G_ij = sum_t |A_it B_tj|
from the oracle):
    |C_gpu - C_oracle| <= 2e-5 * |alpha| * G_ij + 1e-6 * |beta * C_in_ij| + 1e-7
Integer-valued operands: bit-exact (every partial sum is an integer below
2^24, so any summation order gives the same float).
"""
from __future__ import annotations

import numpy as np

REL_G = 2e-5
REL_BETA_C = 1e-6
ABS = 1e-7


def tolerance(G, alpha, beta, C_in):
    return REL_G * abs(alpha) * np.asarray(G) + REL_BETA_C * np.abs(beta * np.asarray(C_in, np.float64)) + ABS


def assert_close(got, want, G, alpha, beta, C_in, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    tol = tolerance(G, alpha, beta, C_in if beta != 0 else 0.0)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]!r} want {want[tuple(i)]!r} "
                           f"tol {tol[tuple(i)]:.3g}" for i in idx)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; {detail}")
    return float((err / tol).max()) if err.size else 0.0


def assert_exact(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    if not np.array_equal(got, want):
        idx = np.argwhere(got != want)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]!r} want {want[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {(got != want).sum()} entries differ; {detail}")


def assert_close_blocked(got, want, G, alpha, beta, C_in, what="", block=1024):
    """assert_close over row blocks of `block` rows (bounds the float64
    temporaries of an 8192 x 8192 comparison); returns the largest err/tol."""
    worst = 0.0
    for r0 in range(0, np.shape(got)[0], block):
        sl = slice(r0, r0 + block)
        cin = C_in[sl] if beta != 0 else 0.0
        worst = max(worst, assert_close(got[sl], want[sl], G[sl], alpha, beta, cin,
                                        f"{what} rows {r0}.."))
    return worst

"""CPU oracle for single-precision GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it,
and it shares no code with the HIP path.

The arithmetic lives in ``oracle_sgemm.c`` (plain C, double accumulation,
loop over the definition C_ij = sum_t A_it * B_tj of page "GEMM优化原理",
section 问题定义, eq. 1, scaled as alpha * S + beta * C_in).  This module only
compiles that file with gcc and marshals numpy arrays to it.

All functions take the operands as flat or 2-D C-contiguous float32 numpy
arrays in row-major storage with an explicit leading dimension, mirroring the
C interface: A_it = A[i*lda + t], B_tj = B[t*ldb + j], C_ij = C[i*ldc + j];
with ``trans_a`` / ``trans_b`` an operand is stored transposed instead:
A_it = A[t*lda + i] (A is k x m), B_tj = B[j*ldb + t] (B is n x k).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle_sgemm.c"
SRC_REDUCE = HERE / "oracle_reduce.c"
LIB = HERE / "liboracle_sgemm.so"

_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_vp = ctypes.c_void_p


def build(src: Path | str = SRC, out: Path | str = LIB,
          src_reduce: Path | str = SRC_REDUCE) -> Path:
    """Compile the oracle (GEMM and array-sum sources) with gcc into a shared
    library (always rebuilds)."""
    out = Path(out)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           str(src), str(src_reduce), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def default_threads() -> int:
    """Host threads available to this process."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover - non-Linux
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


def _f32_flat(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.float32:
        raise TypeError(f"{name} must be float32, got {x.dtype}")
    if not x.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    return x.reshape(-1)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path | str = LIB):
        path = Path(path)
        if not path.exists():
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(str(path))
        rows_args = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64,
                     _i64, _vp, _vp, _vp, ctypes.c_int]
        lib.oracle_sgemm_rows_ex.restype = ctypes.c_int
        lib.oracle_sgemm_rows_ex.argtypes = [ctypes.c_int, ctypes.c_int] + rows_args
        lib.oracle_sum.restype = ctypes.c_int
        lib.oracle_sum.argtypes = [_i64, _vp, _vp, _vp]
        points_args = [_i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64,
                       _i64, _vp, _vp, _vp, _vp, _vp]
        lib.oracle_sgemm_points_ex.restype = ctypes.c_int
        lib.oracle_sgemm_points_ex.argtypes = [ctypes.c_int, ctypes.c_int] + points_args
        self.lib = lib

    # -- whole matrix / selected rows ------------------------------------
    def sgemm(self, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, *,
              rows=None, want_s=False, want_g=False, threads=None,
              trans_a=False, trans_b=False):
        """Returns dict(C=updated copy of C, S=..., G=...).

        With ``rows`` (a sequence of row indices) only those rows of the
        returned C are recomputed, and S / G have one row per listed index.
        ``C`` may be None when beta == 0 (a zero matrix of m x ldc is used).
        """
        Af = _f32_flat(np.ascontiguousarray(A), "A") if A is not None else None
        Bf = _f32_flat(np.ascontiguousarray(B), "B") if B is not None else None
        if C is None:
            C = np.zeros(max(m, 0) * max(ldc, 1), dtype=np.float32)
        Cout = _f32_flat(np.array(C, dtype=np.float32, copy=True, order="C"), "C")
        nrows = m if rows is None else len(rows)
        rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        S = np.empty((nrows, n), dtype=np.float64) if want_s else None
        G = np.empty((nrows, n), dtype=np.float64) if want_g else None
        t = default_threads() if threads is None else int(threads)
        rc = self.lib.oracle_sgemm_rows_ex(
            int(bool(trans_a)), int(bool(trans_b)),
            m, n, k, alpha, _ptr(Af), lda, _ptr(Bf), ldb, beta, _ptr(Cout), ldc,
            nrows, _ptr(rows_arr), _ptr(S), _ptr(G), t)
        if rc != 0:
            raise ValueError(f"oracle_sgemm_rows_ex returned {rc}")
        return {"C": Cout.reshape(np.shape(C)) if np.ndim(C) == 2 else Cout,
                "S": S, "G": G}

    # -- sum of an array ------------------------------------------------
    def sum(self, x):
        """(sum, sum of absolute values) of a float32 array, in double."""
        xf = _f32_flat(np.ascontiguousarray(x), "x")
        s = ctypes.c_double()
        a = ctypes.c_double()
        rc = self.lib.oracle_sum(xf.size, _ptr(xf), ctypes.byref(s), ctypes.byref(a))
        if rc != 0:
            raise ValueError(f"oracle_sum returned {rc}")
        return s.value, a.value

    # -- single entries -------------------------------------------------
    def points(self, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ii, jj, *,
               trans_a=False, trans_b=False):
        """Entries (ii[p], jj[p]); returns dict(C=float32[p], S=..., G=...)."""
        Af = _f32_flat(np.ascontiguousarray(A), "A")
        Bf = _f32_flat(np.ascontiguousarray(B), "B")
        Cf = None if C is None else _f32_flat(np.ascontiguousarray(C), "C")
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        if ii.shape != jj.shape:
            raise ValueError("ii and jj differ in length")
        out = np.empty(ii.size, dtype=np.float32)
        S = np.empty(ii.size, dtype=np.float64)
        G = np.empty(ii.size, dtype=np.float64)
        if Cf is None and beta != 0:
            raise ValueError("beta != 0 needs C")
        rc = self.lib.oracle_sgemm_points_ex(
            int(bool(trans_a)), int(bool(trans_b)),
            m, n, k, alpha, _ptr(Af), lda, _ptr(Bf), ldb, beta, _ptr(Cf), ldc,
            ii.size, _ptr(ii), _ptr(jj), _ptr(out), _ptr(S), _ptr(G))
        if rc != 0:
            raise ValueError(f"oracle_sgemm_points_ex returned {rc}")
        return {"C": out, "S": S, "G": G}


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``oracle_sgemm.c`` next to this file."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default

"""Seeded synthetic operands for the single-precision GEMM workloads.

This module is the only code that both the CPU oracle's tests and the HIP
path's tests/benchmark share.  It draws random matrices and lays them out in
padded row-major storage; it holds none of the GEMM arithmetic.

Recipe (stated once, used everywhere):
  * generator: ``numpy.random.default_rng([workload_id, operand])`` with
    operand 0 = A, 1 = B, 2 = C (the input C); integer-valued twins add a
    third word 1: ``default_rng([workload_id, operand, 1])``;
  * "uniform": float32 values ``2*u - 1`` with u uniform in [0, 1) drawn as
    float32, i.e. uniform on [-1, 1);
  * "normal": float32 standard normal N(0, 1);
  * "int3": integers drawn uniformly from {-3, ..., 3}, stored as float32;
  * storage: a (rows, ld) float32 array; columns at index >= the logical
    width are padding, filled with NaN for A and B and with a fixed sentinel
    for C, so that any read or write of a pad shows up in a test.

The five workloads are the ones the GEMM is measured on: a small 256^3 case,
the 2048^3 size of the worked example on page "GEMM优化原理" (section
一个具体的例子) and of the timing on page "gemm优化" (section 最终测试结果),
8192^3 with alpha/beta, a shape with ragged tails and padded leading
dimensions, and a K-heavy 512 x 512 x 262144 product for split-K.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

C_SENTINEL = np.float32(-12345.5)  # written into C's pad columns


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    m: int
    n: int
    k: int
    lda: int
    ldb: int
    ldc: int
    dist: str            # distribution of A and B
    dist_c: str | None   # distribution of the input C (None: C not read)
    alpha: float
    beta: float
    splitk: bool = False

    @property
    def flops(self) -> float:
        """2*m*n*k, the operation count used for TFLOP/s."""
        return 2.0 * self.m * self.n * self.k

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload(0, "sgemm_256x256x256", 256, 256, 256, 256, 256, 256,
             "uniform", None, 1.0, 0.0),
    Workload(1, "sgemm_2048x2048x2048", 2048, 2048, 2048, 2048, 2048, 2048,
             "uniform", None, 1.0, 0.0),
    Workload(2, "sgemm_8192x8192x8192_ab", 8192, 8192, 8192, 8192, 8192, 8192,
             "normal", "normal", 1.5, 0.5),
    Workload(3, "sgemm_tails_3001x4997x1023", 3001, 4997, 1023, 1028, 5000, 5004,
             "uniform", None, 1.0, 0.0),
    Workload(4, "sgemm_splitk_512x512x262144", 512, 512, 262144, 262144, 512, 512,
             "uniform", None, 1.0, 0.0, splitk=True),
    # an under-filled grid (144 tiles of 128 x 128 on 256 CUs): the split-K
    # entry's plan runs it on the stream-K schedule
    Workload(5, "sgemm_1536x1536x4096", 1536, 1536, 4096, 4096, 1536, 1536,
             "uniform", None, 1.0, 0.0),
    # a small grid with a short k: the split-K entry's plan runs the
    # 64 x 64 x 32 tile on stream-K with one workgroup per CU
    Workload(20, "sgemm_1536x1536x1024", 1536, 1536, 1024, 1024, 1536, 1536,
             "uniform", None, 1.0, 0.0),
]


def workload(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)


def draw(rng: np.random.Generator, rows: int, cols: int, dist: str) -> np.ndarray:
    """rows x cols float32 values from one of the named distributions."""
    if dist == "uniform":
        u = rng.random((rows, cols), dtype=np.float32)
        u *= np.float32(2.0)
        u -= np.float32(1.0)
        return u
    if dist == "normal":
        return rng.standard_normal((rows, cols), dtype=np.float32)
    if dist == "int3":
        return rng.integers(-3, 4, size=(rows, cols), dtype=np.int8).astype(np.float32)
    if dist == "ones":
        return np.ones((rows, cols), dtype=np.float32)
    if dist == "zeros":
        return np.zeros((rows, cols), dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def padded(values: np.ndarray, ld: int, pad: float) -> np.ndarray:
    """Place a rows x cols block into a rows x ld array, pads set to `pad`."""
    rows, cols = values.shape
    if ld < cols:
        raise ValueError("leading dimension smaller than the width")
    out = np.empty((rows, max(ld, 1)), dtype=np.float32)
    out[:, :cols] = values
    out[:, cols:] = pad
    return out


def matrix(wid: int, operand: int, rows: int, cols: int, ld: int, dist: str,
           integer_twin: bool = False, pad: float | None = None) -> np.ndarray:
    seed = [wid, operand, 1] if integer_twin else [wid, operand]
    rng = np.random.default_rng(seed)
    if pad is None:
        pad = C_SENTINEL if operand == 2 else np.float32(np.nan)
    return padded(draw(rng, rows, cols, dist), ld, pad)


def operands(w: Workload, integer_twin: bool = False):
    """(A, B, C) as padded float32 arrays for workload `w`.

    C is always returned (pads = sentinel); it holds drawn values only when
    the workload reads C (beta != 0), zeros otherwise.  The integer twin
    draws every operand from "int3" with its own seeds.
    """
    da = "int3" if integer_twin else w.dist
    dc = ("int3" if integer_twin else w.dist_c) if w.dist_c else "zeros"
    A = matrix(w.wid, 0, w.m, w.k, w.lda, da, integer_twin)
    B = matrix(w.wid, 1, w.k, w.n, w.ldb, da, integer_twin)
    C = matrix(w.wid, 2, w.m, w.n, w.ldc, dc, integer_twin)
    return A, B, C


def transposed_storage(M: np.ndarray, cols: int, ld: int, pad=np.float32(np.nan)) -> np.ndarray:
    """Storage of the transpose of the logical block M[:, :cols]: a
    cols x ld array (ld >= M's row count), pads set to `pad`."""
    return padded(np.ascontiguousarray(M[:, :cols].T), ld, pad)


def transposed_ld(rows: int, width: int, ld: int) -> int:
    """Leading dimension for storing a rows-long operand transposed, keeping
    the padding of the as-given layout (ld - width) and, when ld is a
    multiple of 4, that property too."""
    out = rows + (ld - width)
    if ld % 4 == 0:
        out = (out + 3) // 4 * 4
    return max(out, 1)


def operands_ex(w: Workload, trans_a: bool, trans_b: bool, integer_twin: bool = False):
    """(A, lda, B, ldb, C) with the values of operands(w); A is stored k x m
    when trans_a, B is stored n x k when trans_b (NaN pads)."""
    A, B, C = operands(w, integer_twin)
    lda, ldb = w.lda, w.ldb
    if trans_a:
        lda = transposed_ld(w.m, w.k, w.lda)
        A = transposed_storage(A, w.k, lda)
    if trans_b:
        ldb = transposed_ld(w.k, w.n, w.ldb)
        B = transposed_storage(B, w.n, ldb)
    return A, lda, B, ldb, C


def sample_indices(seed, m: int, n: int, count: int):
    """`count` distinct-ish (i, j) positions for sampled checks, always
    including the four corners of the m x n output."""
    rng = np.random.default_rng(seed)
    ii = rng.integers(0, m, size=count, dtype=np.int64)
    jj = rng.integers(0, n, size=count, dtype=np.int64)
    corners_i = np.array([0, 0, m - 1, m - 1], dtype=np.int64)
    corners_j = np.array([0, n - 1, 0, n - 1], dtype=np.int64)
    return np.concatenate([corners_i, ii]), np.concatenate([corners_j, jj])


def sample_rows(seed, m: int, count: int) -> np.ndarray:
    """`count` distinct rows of an m-row output, always including 0 and m-1."""
    if count >= m:
        return np.arange(m, dtype=np.int64)
    rng = np.random.default_rng(seed)
    pick = rng.choice(m, size=count, replace=False).astype(np.int64)
    pick[0] = 0
    if count > 1:
        pick[-1] = m - 1
    return np.unique(pick)


# Array-sum workloads (the reduction of page aerisun.top, section
# "Reduce 的分层归约"): n float32 values, uniform on [-1, 1).
REDUCE_WORKLOADS = {
    "reduce_sum_1048576": (200, 1 << 20),
    "reduce_sum_268435456": (201, 1 << 28),
}


def vector(name_or_n, integer_twin: bool = False, seed_id: int | None = None) -> np.ndarray:
    """The seeded input of a named array-sum workload, or of size n (with
    seed id `seed_id`, default 299)."""
    if isinstance(name_or_n, str):
        wid, n = REDUCE_WORKLOADS[name_or_n]
    else:
        wid, n = (299 if seed_id is None else seed_id), int(name_or_n)
    seed = [wid, 0, 1] if integer_twin else [wid, 0]
    rng = np.random.default_rng(seed)
    return draw(rng, 1, n, "int3" if integer_twin else "uniform").reshape(n)

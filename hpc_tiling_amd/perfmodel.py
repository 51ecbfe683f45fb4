"""Operation counts, algorithmic bytes and roofline bounds for SGEMM.

Host arithmetic only (no GPU), used by the benchmark to turn measured times
into TFLOP/s and roofline fractions.  The formulas are the ones the pages
state; the MI355X constants are AMD's published figures.
"""
from __future__ import annotations

# MI355X (gfx950) published peaks.
CUS = 256
XCDS = 8
PEAK_CLOCK_HZ = 2.4e9
PEAK_FP32_MFMA = 157.3e12      # dense FP32 matrix, 256 FLOP/clk/CU at 2.4 GHz
PEAK_FP32_VECTOR = 157.3e12    # FP32 vector ALUs, 256 FLOP/clk/CU at 2.4 GHz
# The VALU kernel's bound.  Built without packed FP32 instructions, its inner
# loop is plain v_fma_f32 with every operand in a VGPR.  Measured on MI355X,
# such an 8 x 8 register outer product sustains 136-138 TFLOP/s over runs
# (0.87 of 256 FLOP/clk/CU), while FMA chains with an SGPR operand sustain
# 77 (128 FLOP/clk/CU): the full vector rate, not half of it, bounds the loop.
PEAK_FP32_VALU = 157.3e12
PEAK_FP32_VALU_NOTE = ("FP32 vector peak, 256 FLOP/clk/CU x 256 CUs x 2.4 GHz: plain v_fma_f32 "
                       "with VGPR operands issues at that rate (an 8x8 register outer product "
                       "measured 136-138 TFLOP/s on MI355X)")
PEAK_HBM_BYTES = 8.0e12        # HBM3E
ELEM = 4                       # bytes per float


def gemm_flops(m: int, n: int, k: int) -> float:
    """2mnk: one multiply and one add per term of C_ij = sum_t A_it B_tj
    (page "GEMM优化原理", section 问题定义, eq. 1; page aerisun.top counts an
    FMA as 2 FLOPs in section "GEMM 的理想复用与实际访存")."""
    return 2.0 * m * n * k


def tflops(m: int, n: int, k: int, seconds: float, reps: int = 1) -> float:
    """Throughput of `reps` products of m x k by k x n in `seconds`."""
    return gemm_flops(m, n, k) * reps / seconds / 1e12


def ideal_bytes(m: int, n: int, k: int, beta_nonzero: bool = False) -> float:
    """Bytes if every input is read from DRAM once and C written once
    (plus read once when beta != 0): page aerisun.top, section
    "GEMM 的理想复用与实际访存", eq. for I_ideal."""
    return ELEM * (m * k + k * n + m * n * (2 if beta_nonzero else 1))


def ideal_intensity(m: int, n: int, k: int, beta_nonzero: bool = False) -> float:
    """FLOP per byte at ideal reuse; n/6 for a square n^3 product."""
    return gemm_flops(m, n, k) / ideal_bytes(m, n, k, beta_nonzero)


def tile_intensity(bm: int, bn: int) -> float:
    """FLOP per byte of one workgroup tile step: 2 bm bn bk / 4 (bm bk + bk bn)
    = bm bn / (2 (bm + bn)) (page aerisun.top, section
    "Shared Tiling 与 block 内复用")."""
    return bm * bn / (2.0 * (bm + bn))


def tiled_global_reads(m: int, n: int, k: int, bm: int, bn: int) -> float:
    """Elements read from global memory with bm x bn block tiles:
    mnk (1/bm + 1/bn) (page "GEMM优化原理", section 基于 shared memory 计算)."""
    return m * n * k * (1.0 / bm + 1.0 / bn)


def tiled_shared_reads(m: int, n: int, k: int, rm: int, rn: int) -> float:
    """Elements read from shared memory with rm x rn register tiles:
    mnk (1/rm + 1/rn) (page "GEMM优化原理", section 基于 register 计算)."""
    return m * n * k * (1.0 / rm + 1.0 / rn)


def ridge(peak_flops: float, bandwidth: float) -> float:
    """Intensity where the two roofs meet, I* = P_peak / BW (page
    aerisun.top, section "Roofline 与算术强度")."""
    return peak_flops / bandwidth


def roofline(peak_flops: float, bandwidth: float, intensity: float) -> float:
    """Attainable FLOP/s: min(P_peak, BW * I) (same section)."""
    return min(peak_flops, bandwidth * intensity)


def splitk_combine_bytes(m: int, n: int, splits: int, beta_nonzero: bool = False) -> float:
    """Bytes the split-K combine must move: read `splits` partial m x n
    matrices, write C (and read it when beta != 0)."""
    return ELEM * m * n * (splits + 1 + (1 if beta_nonzero else 0))

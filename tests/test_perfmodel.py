"""The benchmark's FLOP / byte / roofline arithmetic against the figures the
pages print (tests/golden/*.txt)."""
from pathlib import Path

import pytest

from hpc_tiling_amd import perfmodel as pm

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rows(name):
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if line and not line.startswith("#"):
            yield line.split()


def test_tflops_formula_reproduces_printed_pairs():
    rows = [r for r in _rows("timings_lightlisten_2048.txt") if r[0] != "label"]
    assert len(rows) == 4
    for label, ms, tf in rows:
        got = pm.tflops(2048, 2048, 2048, float(ms) / 1e3, reps=10_000)
        assert round(got, 3) == pytest.approx(float(tf), abs=0.0015), label


def test_intensity_examples():
    g = {r[0]: float(r[1]) for r in _rows("intensity_examples.txt")}
    # 64x64 tile, step 64: bytes = 4 (64*64 + 64*64), flops = 2 * 64^3
    bytes_ = 4 * (64 * 64 + 64 * 64)
    flop = pm.gemm_flops(64, 64, 64)
    assert bytes_ == g["tile64_bytes"] and flop == g["tile64_flop"]
    assert pm.tile_intensity(64, 64) == g["tile64_intensity"] == flop / bytes_
    assert bytes_ / 256 == g["tile64_thread_bytes"]
    assert 64 ** 3 / 256 == g["tile64_thread_fma"]
    r = pm.ridge(g["rtx4070tis_peak_tflops"] * 1e12, g["rtx4070tis_bw_gbs"] * 1e9)
    assert r == pytest.approx(65.6, abs=0.05)
    assert abs(r - g["rtx4070tis_ridge_printed"]) < 0.25   # the page's rounding slip
    for n in (6, 256, 2048, 8192):
        assert pm.ideal_intensity(n, n, n) == pytest.approx(n / g["ideal_intensity_divisor"])
    # one output per thread: 2K FLOP over 2K loads + 1 store of 4 bytes
    K = 4096
    assert 2 * K / (8 * K + 4) == pytest.approx(g["naive_intensity"], rel=1e-3)


def test_read_counts_match_worked_example():
    g = {r[0]: int(r[1]) for r in _rows("worked_example_2048.txt")}
    m, n, k = g["m"], g["n"], g["k"]
    per_block_global = g["big_iterations"] * (g["a_elements_per_big_iteration"]
                                               + g["b_elements_per_big_iteration"])
    assert g["workgroups"] * per_block_global == pytest.approx(
        pm.tiled_global_reads(m, n, k, g["tile_m"], g["tile_n"]))
    # shared reads: every thread reads r_m + r_n values per small iteration
    shared = (g["workgroups"] * g["threads"] * g["big_iterations"] * g["small_iterations"]
              * (g["micro_m"] + g["micro_n"]))
    assert shared == pytest.approx(pm.tiled_shared_reads(m, n, k, g["micro_m"], g["micro_n"]))
    assert g["fma_per_small_iteration"] * g["small_iterations"] * g["big_iterations"] \
        * g["threads"] * g["workgroups"] == m * n * k


def test_roofline_and_mi355x_ridge():
    assert pm.roofline(10.0, 2.0, 3.0) == 6.0
    assert pm.roofline(10.0, 2.0, 30.0) == 10.0
    assert pm.ridge(pm.PEAK_FP32_MFMA, pm.PEAK_HBM_BYTES) == pytest.approx(19.66, abs=0.01)
    assert pm.PEAK_FP32_MFMA == pytest.approx(pm.CUS * 256 * pm.PEAK_CLOCK_HZ, rel=0.01)
    assert pm.PEAK_FP32_VECTOR == pytest.approx(pm.CUS * 256 * pm.PEAK_CLOCK_HZ, rel=0.01)
    assert pm.splitk_combine_bytes(512, 512, 64) == 4 * 512 * 512 * 65

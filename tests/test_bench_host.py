"""Host logic of bench.py, without a GPU: the one-GPU refusal, the trial
statistics, the rocprofv3 summaries the profiles are made from, and the rule
that recorded traffic is reported only for the sources it was measured on."""
import csv
import importlib.util
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused(bench, capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_trial_stats(bench):
    # three trials of 10 steps: 1.0, 1.2 and 1.1 ms per step
    st = bench.trial_stats([0.010, 0.012, 0.011], 10, 2e9)
    assert st["count"] == 3 and st["steps_each"] == 10
    assert st["ms_per_step_median"] == pytest.approx(1.1)
    assert (st["ms_per_step_min"], st["ms_per_step_max"]) == pytest.approx((1.0, 1.2))
    assert st["tflops_median"] == pytest.approx(2e9 / 1.1e-3 / 1e12)
    assert st["tflops_max"] == pytest.approx(2e9 / 1.0e-3 / 1e12)
    assert st["tflops_min"] == pytest.approx(2e9 / 1.2e-3 / 1e12)


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_trace_takes_the_last_matching_dispatches(bench, tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    # (name, start ns, end ns), out of order in the file
    rows = [("other_kernel", 0, 5_000_000),
            ("void mi::sgemm_mfma_kernel<...>", 3_000, 303_000),     # 300 us, last
            ("void mi::sgemm_mfma_kernel<...>", 1_000, 101_000),     # 100 us, first
            ("void mi::sgemm_mfma_kernel<...>", 2_000, 202_000)]     # 200 us
    _write_csv(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    d = bench.summarize_trace(str(p), "sgemm_mfma_kernel", 2, flop=1e9)
    assert d["dispatches_in_trace"] == 3 and d["dispatches_used"] == 2
    assert d["avg_us"] == pytest.approx(250.0)
    assert (d["min_us"], d["max_us"]) == pytest.approx((200.0, 300.0))
    assert d["tflops_at_avg"] == pytest.approx(1e9 / 250e-6 / 1e12)
    assert d["frac_of_fp32_peak_at_avg"] == pytest.approx(d["tflops_at_avg"] / 157.3)
    d = bench.summarize_trace(str(p), "sgemm_mfma_kernel", 0, nbytes=8e6)
    assert d["dispatches_used"] == 3 and d["avg_us"] == pytest.approx(200.0)
    assert d["gb_per_s_at_avg"] == pytest.approx(40.0)


def test_summarize_counters_sums_rows_of_a_dispatch(bench, tmp_path):
    p = tmp_path / "run_counter_collection.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"]
    rows = []
    # dispatch d of the kernel: FETCH_SIZE reported in two rows (e.g. two
    # instances) of d and 2d KiB; another kernel in between
    for d in (1, 2, 3):
        rows.append((d, "sgemm_mfma_kernel", "FETCH_SIZE", d, 64))
        rows.append((d, "sgemm_mfma_kernel", "FETCH_SIZE", 2 * d, 64))
        rows.append((10 + d, "copyBuffer", "FETCH_SIZE", 1000, 1))
    _write_csv(p, hdr, rows)
    s = bench.summarize_counters(str(p), "sgemm_mfma_kernel", 2)
    assert s["dispatches_in_file"] == 3 and s["dispatches_used"] == 2
    assert s["mean"]["FETCH_SIZE"] == pytest.approx((6 + 9) / 2)
    assert s["resources_of_last_dispatch"]["Grid_Size"] == "64"


def test_traffic_is_reported_only_for_its_sources(bench, tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_mfma_w.txt").write_text(
        "# header: not data\nsource_digest: abc123\nhbm_bytes_per_launch: 1.5e+08\n")
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setattr(bench, "source_digest", lambda: "abc123")
    assert bench.read_traffic("mfma", "w") == pytest.approx(1.5e8)
    monkeypatch.setattr(bench, "source_digest", lambda: "other")
    assert bench.read_traffic("mfma", "w") is None
    assert bench.read_traffic("mfma", "missing") is None


def test_source_digest_follows_every_kernel_source(bench, tmp_path, monkeypatch):
    import shutil
    for sub in ("hpc_tiling_amd/csrc", "include"):
        shutil.copytree(ROOT / sub, tmp_path / sub)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    d0 = bench.source_digest()
    assert len(d0) == 16 and d0 == bench.source_digest()
    for f in [*sorted((tmp_path / "hpc_tiling_amd/csrc").glob("*")),
              *sorted((tmp_path / "include").glob("*.h"))]:
        text = f.read_bytes()
        f.write_bytes(text + b"\n")
        assert bench.source_digest() != d0, f.name
        f.write_bytes(text)
    assert bench.source_digest() == d0

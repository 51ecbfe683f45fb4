#!/usr/bin/env python3
"""SGEMM benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials T]
                    [--workload NAME] [--kernel KIND]

One step is one call of the hot path (C = alpha*A*B + beta*C through the C
ABI) on seeded synthetic operands already resident in HBM.  W untimed steps
(continued until the clock has settled), then T trials of exactly K steps,
each timed with HIP events on the stream the kernels run on, between
synchronisations.  Prints ONE JSON line: throughput in TFLOP/s (2mnk per
step) of the median trial, the spread of the trials, the GPU clocks before,
during and after the timed trials, the roofline object of the GEMM kernel
(the only kernel a step of the default workload launches, so its average
duration is the step time), the CPU oracle timed on a bounded sample of the
same workload, and secondary measurements of the other workloads and of the
split-K combine kernel on its own.

Two helpers turn rocprofv3 output of a run of this script into the figures
under profiles/ (averaged over the timed dispatches, the last T*K ones):
    python bench.py --summarize-trace kernel_trace.csv --match NAME --last N
    python bench.py --summarize-counters counter_collection.csv --match NAME --last N

Only the CPU-baseline leg imports the oracle.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

DEFAULT_WORKLOAD = "sgemm_2048x2048x2048"
METRIC = "SGEMM TFLOPS at 2048^3 and 8192^3 FP32; % of MI355X FP32 peak"


def source_digest() -> str:
    """Hash of the kernel sources and header; traffic counters recorded for
    another digest describe other code and are not reported."""
    h = hashlib.sha256()
    files = sorted((ROOT / "hpc_tiling_amd" / "csrc").glob("*")) + sorted((ROOT / "include").glob("*.h"))
    for f in files:
        h.update(f.name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt, if
    it was measured on the current sources."""
    p = ROOT / "profiles" / f"traffic_{kernel}_{workload}.txt"
    if not p.exists():
        return None
    kv = {}
    for line in p.read_text().splitlines():
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# GPU clocks
# ---------------------------------------------------------------------------
def mclk_mhz():
    """(memory clock in MHz, None) from the driver's GPU metrics table (amdsmi),
    or (None, reason).  The same table's graphics clock reads an idle value
    between launches, so the core clock is measured on the GPU instead
    (mi_clock_probe)."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        return float(amdsmi.amdsmi_get_gpu_metrics_info(h)["current_uclk"]), None
    except Exception as e:  # noqa: BLE001 - any failure means "not recorded"
        return None, f"{type(e).__name__}: {e}"


def clock_summary(mhz):
    return {"mean": statistics.fmean(mhz), "min": min(mhz), "max": max(mhz),
            "per_xcd": [round(x, 1) for x in mhz]}


# ---------------------------------------------------------------------------
# Steps and timing
# ---------------------------------------------------------------------------
def make_step(kind, w, Av, Bv, Cv, ws):
    import hpc_tiling_amd as hta
    alpha, beta = w.alpha, w.beta
    if kind == "mfma":
        return lambda: hta.sgemm(Av, Bv, Cv, alpha, beta)
    if kind == "valu":
        return lambda: hta.sgemm_valu(Av, Bv, Cv, alpha, beta)
    if kind == "splitk":
        return lambda: hta.sgemm_splitk(Av, Bv, Cv, alpha, beta, splits=0, workspace=ws)
    if kind == "splitk_atomic":
        return lambda: hta.sgemm_splitk_atomic(Av, Bv, Cv, alpha, beta, splits=0)
    if kind.startswith("mfma_cfg"):
        cfg = int(kind[len("mfma_cfg"):])
        return lambda: hta.sgemm(Av, Bv, Cv, alpha, beta, config=cfg)
    if kind == "mfma_raw":
        # the C entry point with its arguments prepared once: for products
        # small enough that the Python helper's checks take longer than the
        # kernel
        import torch
        (ta, tb, m, n, k, pa, lda, pb, ldb), C, pc, ldc, _ = hta._prepare_ex(Av, Bv, Cv, beta)
        fn = hta.lib.mi_sgemm_ex
        args = (ta, tb, m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc,
                torch.cuda.current_stream().cuda_stream)
        if fn(*args) != hta.SUCCESS:
            raise RuntimeError("mi_sgemm_ex failed")
        return lambda: fn(*args)
    if kind.startswith("streamk_c"):
        # forced stream-K schedule: streamk_c<config>_g<grid>
        cfg, grid = (int(x) for x in kind[len("streamk_c"):].split("_g"))
        return lambda: hta.sgemm_streamk(Av, Bv, Cv, alpha, beta, grid=grid, workspace=ws,
                                         config=cfg)
    if kind.startswith("mfma_x"):
        # forced workgroup order: mfma_x<xcd_remap>g<group_m>, e.g. mfma_x0g1
        x, g = kind[len("mfma_x"):].split("g")
        order = (int(x), int(g))
        return lambda: hta.sgemm(Av, Bv, Cv, alpha, beta, order=order)
    raise ValueError(kind)


# Kind suffixes for operands stored transposed (A^T is k x m, B^T is n x k);
# the stored matrices are passed as transposed (column-major) views.
TRANS_SUFFIXES = {"_nt": (False, True), "_tn": (True, False), "_tt": (True, True)}


def setup(w, kind):
    import torch
    import hpc_tiling_amd as hta
    import synth
    ta = tb = False
    for suffix, flags in TRANS_SUFFIXES.items():
        if kind.endswith(suffix):
            kind = kind[:-len(suffix)]
            ta, tb = flags
    A, _, B, _, C = synth.operands_ex(w, ta, tb)
    dev = torch.device("cuda:0")
    Ad, Bd, Cd = (torch.from_numpy(x).to(dev) for x in (A, B, C))
    Av = Ad[:, :w.m].t() if ta else Ad[:, :w.k]
    Bv = Bd[:, :w.k].t() if tb else Bd[:, :w.n]
    ws = None
    if kind == "splitk":
        ws = hta.splitk_workspace(w.m, w.n, w.k, 0, device=dev)
    elif kind.startswith("streamk_c"):
        cfg, grid = (int(x) for x in kind[len("streamk_c"):].split("_g"))
        ws = hta.streamk_workspace(w.m, w.n, w.k, grid, device=dev, config=cfg)
    torch.cuda.synchronize()
    return (A, B, C), (Ad, Bd, Cd), make_step(kind, w, Av, Bv, Cd[:, :w.n], ws)


SETTLE_S = 0.2


def warm(step, warmup, settle_s=SETTLE_S):
    """`warmup` untimed calls; after an idle spell the GPU clock needs about
    30 ms of load to reach its steady value, so untimed calls continue (in
    batches of 10) until at least `settle_s` seconds of back-to-back calls have
    run.  Returns the number of extra calls."""
    import torch
    start = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - start < settle_s:
        for _ in range(10):
            step()
        extra += 10
        torch.cuda.synchronize()
    return extra


def time_trials(step, steps, trials, probes=None):
    """Seconds of each of `trials` runs of exactly `steps` calls, measured with
    events on the current stream (the stream the kernels are launched on).
    The runs follow each other on the GPU with no gap (an event between two
    runs ends one and starts the next); the whole timed region is bracketed
    by synchronisations.  `probes` = (before, after) ClockProbe objects
    launched right before the first and right after the last run.  Also
    returns the host seconds spent issuing the calls."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
    torch.cuda.synchronize()
    if probes:
        probes[0].launch()
    h0 = time.perf_counter()
    ev[0].record(stream)
    for t in range(trials):
        for _ in range(steps):
            step()
        ev[t + 1].record(stream)
    host = time.perf_counter() - h0
    if probes:
        probes[1].launch()
    torch.cuda.synchronize()
    return [ev[t].elapsed_time(ev[t + 1]) / 1e3 for t in range(trials)], host / trials


def trial_stats(secs, steps, flops):
    ms = sorted(1e3 * s / steps for s in secs)
    med = statistics.median(ms)
    return {"count": len(ms), "steps_each": steps, "ms_per_step_median": med,
            "ms_per_step_min": ms[0], "ms_per_step_max": ms[-1],
            "tflops_median": flops / (med * 1e-3) / 1e12,
            "tflops_max": flops / (ms[0] * 1e-3) / 1e12,
            "tflops_min": flops / (ms[-1] * 1e-3) / 1e12}


def cpu_baseline(w, host, budget_s):
    """The oracle on whole output rows of the same workload, as many rows as
    fit the time budget (estimated from a first small batch)."""
    import oracle
    import synth
    A, B, C = host
    orc = oracle.get()
    threads = oracle.default_threads()
    probe = synth.sample_rows([w.wid, 1234], w.m, min(w.m, max(threads, 8)))
    t0 = time.perf_counter()
    orc.sgemm(w.m, w.n, w.k, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, rows=probe,
              want_g=True, threads=threads)
    per_row = (time.perf_counter() - t0) / len(probe)
    nrows = int(min(w.m, max(len(probe), budget_s / max(per_row, 1e-9))))
    nrows = max(threads, (nrows // threads) * threads) if nrows < w.m else w.m
    rows = synth.sample_rows([w.wid, 4321], w.m, nrows)
    # when every row fits the budget, whole passes are repeated until it is spent
    passes = 0
    t0 = time.perf_counter()
    while True:
        orc.sgemm(w.m, w.n, w.k, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, rows=rows,
                  want_g=True, threads=threads)
        passes += 1
        if nrows < w.m or time.perf_counter() - t0 >= budget_s or passes >= 200:
            break
    dt = time.perf_counter() - t0
    used = int(min(threads, len(rows)))
    flops = 2.0 * passes * len(rows) * w.n * w.k
    what = (f"{len(rows)} of {w.m} output rows" if len(rows) < w.m
            else f"all {w.m} output rows, {passes} pass(es)")
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
        "sample": (f"{what} of {w.name} (all {w.n} columns, full k={w.k}); FP64 "
                   f"accumulation, also summing |A_it B_tj|; {dt:.2f} s"),
        "seconds": dt, "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def timed_calls(step, seconds):
    """(calls, seconds per call on the GPU, host seconds per call) of about
    `seconds` of back-to-back calls, after a short warmup."""
    warm(step, 2, 0.02)
    probe, _ = time_trials(step, 2, 1)
    n = max(3, min(5000, int(seconds / max(probe[0] / 2, 1e-6))))
    # (the operands of the next workload take seconds to generate, with the
    # GPU idle: settle as long as for the headline)
    warm(step, 5, SETTLE_S)
    secs, host = time_trials(step, n, 1)
    return n, secs[0] / n, host / n


def secondary(kinds_workloads, seconds=0.25):
    """TFLOP/s of other (kernel, workload) pairs, each timed over about
    `seconds` of back-to-back calls.  host_us_per_call is the time the host
    spends issuing one call; where it is not below the GPU time per call the
    line measures host dispatch, not the kernel, and says so."""
    import torch
    import synth
    from hpc_tiling_amd import perfmodel as pm
    out = []
    for kind, name in kinds_workloads:
        w = synth.workload(name)
        host, dev, step = setup(w, kind)
        n, per_call, host_per_call = timed_calls(step, seconds)
        tf = w.flops / per_call / 1e12
        rec = {"workload": name, "kernel": kind, "calls": n, "ms_per_call": 1e3 * per_call,
               "tflops": tf, "frac_of_fp32_peak": tf * 1e12 / pm.PEAK_FP32_MFMA,
               "host_us_per_call": 1e6 * host_per_call}
        if host_per_call >= 0.9 * per_call:
            rec["note"] = ("host-bound: issuing a call takes about as long as the GPU work, "
                           "so this measures dispatch, not the kernel")
        out.append(rec)
        del host, dev, step
        torch.cuda.empty_cache()
    return out


def cold_secondary(kind="mfma", name="sgemm_2048x2048x2048", calls=40, flush_mib=512):
    """One call at a time, each timed alone between HIP events, with the
    operands out of every cache (a cold-cache run): before
    each call a 512 MiB buffer, twice the 256 MB last-level cache, is
    overwritten on the same stream.  The same single-call timing without the
    flush is reported beside it, so that the difference is what the cold
    caches cost (a single call also pays its own launch, which back-to-back
    calls overlap)."""
    import torch
    import synth
    from hpc_tiling_amd import perfmodel as pm
    w = synth.workload(name)
    host, dev, step = setup(w, kind)
    buf = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda:0")
    warm(step, 3, 0.02)

    def single_calls(flush):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        for e0, e1 in evs:
            if flush:
                buf.fill_(1.0)
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)

    rec = {"workload": name + " cold", "kernel": kind, "calls": calls,
           "flush": f"{flush_mib} MiB overwritten before each call"}
    for label, flush in (("cold", True), ("warm_single", False)):
        secs = single_calls(flush)
        med = secs[len(secs) // 2]
        rec[label] = {"ms_per_call_median": 1e3 * med, "ms_per_call_min": 1e3 * secs[0],
                      "ms_per_call_max": 1e3 * secs[-1], "tflops": w.flops / med / 1e12,
                      "frac_of_fp32_peak": w.flops / med / pm.PEAK_FP32_MFMA}
    del host, dev, step, buf
    torch.cuda.empty_cache()
    return rec


def combine_secondary(name="sgemm_splitk_512x512x262144", seconds=0.25):
    """The split-K combine kernel alone, at the slice count the automatic
    plan uses for `name`: GB/s of its bytes 4 m n (S + 1) (S partial
    matrices read, C written) and the fraction of the 8 TB/s HBM roofline."""
    import torch
    import hpc_tiling_amd as hta
    import synth
    from hpc_tiling_amd import perfmodel as pm
    w = synth.workload(name)
    plan = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, w.m, w.n, w.k, 0)
    S = plan["splits"]
    mn = w.m * w.n
    slice_ = (mn + 63) // 64 * 64
    g = torch.Generator(device="cpu").manual_seed(4)
    parts = (torch.rand((S, slice_), generator=g) * 2 - 1).to("cuda")
    C = torch.empty((w.m, w.n), device="cuda")
    # the raw entry point with its arguments prepared once: the Python helper
    # costs more host time per call than the kernel takes
    fn = hta.lib.mi_sgemm_splitk_combine
    args = (w.m, w.n, S, parts.data_ptr(), slice_, 1.0, 0.0, C.data_ptr(), w.n,
            torch.cuda.current_stream().cuda_stream)
    if fn(*args) != hta.SUCCESS:
        raise RuntimeError("mi_sgemm_splitk_combine failed")
    step = lambda: fn(*args)
    n, per_call, host_per_call = timed_calls(step, seconds)
    nbytes = pm.splitk_combine_bytes(w.m, w.n, S)
    gbs = nbytes / per_call / 1e9
    res = {"workload": f"{name} combine, S={S}", "kernel": "splitk_combine_kernel",
           "calls": n, "us_per_call": 1e6 * per_call, "bytes_per_call": nbytes, "gb_per_s": gbs,
           "frac_of_hbm_peak": gbs * 1e9 / pm.PEAK_HBM_BYTES,
           "host_us_per_call": 1e6 * host_per_call,
           "timing": "HIP events over back-to-back launches of the combine alone"}
    del parts, C
    torch.cuda.empty_cache()
    return res


def valu_calibration(workgroups=256 * 32, iters=2000, launches=10):
    """TFLOP/s of the two FMA loops of mi_fma_rate_probe (8 waves per SIMD):
    the register outer product shaped like the VALU kernel's inner loop, and
    FMA chains with scalar-register operands."""
    import torch
    import hpc_tiling_amd as hta
    from hpc_tiling_amd import perfmodel as pm
    out = torch.empty(256 * workgroups, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    res = {}
    for loop, name, flop in ((0, "outer_product_8x8_vgpr", 136), (1, "chains_sgpr_operand", 256)):
        launch = lambda: hta.mi_fma_rate_probe(loop, out.data_ptr(), workgroups, iters, s.cuda_stream)
        for _ in range(3):
            if launch() != hta.SUCCESS:
                raise RuntimeError("mi_fma_rate_probe failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(launches):
            launch()
        e1.record(s)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / launches
        tf = flop * iters * 256.0 * workgroups / sec / 1e12
        res[name] = {"us_per_launch": 1e6 * sec, "tflops": tf,
                     "frac_of_fp32_vector_peak": tf * 1e12 / pm.PEAK_FP32_VECTOR,
                     "flop_per_launch": flop * iters * 256.0 * workgroups}
    return res


def reduce_secondary(name="reduce_sum_268435456", seconds=0.25):
    """The array sum on its largest workload: GB/s of algorithmic bytes (4n)
    and the fraction of the 8 TB/s HBM roofline."""
    import torch
    import hpc_tiling_amd as hta
    import synth
    from hpc_tiling_amd import perfmodel as pm
    x = torch.from_numpy(synth.vector(name)).to("cuda")
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(hta.mi_reduce_sum_workspace_bytes(x.numel()), 4), dtype=torch.uint8,
                     device="cuda")
    step = lambda: hta.reduce_sum(x, out=out, workspace=ws)
    n, per_call, host_per_call = timed_calls(step, seconds)
    gbs = 4.0 * x.numel() / per_call / 1e9
    res = {"workload": name, "kernel": "reduce_sum", "calls": n, "us_per_call": 1e6 * per_call,
           "gb_per_s": gbs, "frac_of_hbm_peak": gbs * 1e9 / pm.PEAK_HBM_BYTES,
           "host_us_per_call": 1e6 * host_per_call}
    del x, ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# rocprofv3 output -> profile figures
# ---------------------------------------------------------------------------
def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_trace(path, match, last, flop=None, nbytes=None):
    """Duration statistics of the last `last` dispatches whose kernel name
    contains `match` in a rocprofv3 kernel_trace.csv (--kernel-trace), and
    the TFLOP/s or GB/s they imply for `flop` / `nbytes` per dispatch."""
    rows = [r for r in _rows(path) if match in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    sel = rows[-last:] if last else rows
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
    out = {"kernel_match": match, "dispatches_in_trace": len(rows), "dispatches_used": len(sel),
           "avg_us": statistics.fmean(us), "median_us": statistics.median(us),
           "min_us": min(us), "max_us": max(us)}
    if flop:
        out["tflops_at_avg"] = flop / (out["avg_us"] * 1e-6) / 1e12
        out["frac_of_fp32_peak_at_avg"] = out["tflops_at_avg"] / 157.3
    if nbytes:
        out["gb_per_s_at_avg"] = nbytes / (out["avg_us"] * 1e-6) / 1e9
        out["frac_of_hbm_peak_at_avg"] = out["gb_per_s_at_avg"] / 8000.0
    names = sorted({r["Kernel_Name"] for r in sel})
    out["kernel_names"] = names[:4]
    return out


def summarize_counters(path, match, last):
    """Mean of every counter over the last `last` dispatches whose kernel name
    contains `match` in a rocprofv3 counter_collection.csv (--pmc)."""
    per_dispatch = {}
    resources = {}
    for r in _rows(path):
        if match not in r["Kernel_Name"]:
            continue
        d = per_dispatch.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        resources = {k: r[k] for k in ("Kernel_Name", "Grid_Size", "Workgroup_Size", "VGPR_Count",
                                       "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size",
                                       "Scratch_Size") if k in r}
    ids = sorted(per_dispatch)
    sel = ids[-last:] if last else ids
    names = sorted({c for i in sel for c in per_dispatch[i]})
    return {"kernel_match": match, "dispatches_in_file": len(ids), "dispatches_used": len(sel),
            "resources_of_last_dispatch": resources,
            "mean": {c: statistics.fmean(per_dispatch[i].get(c, 0.0) for i in sel)
                     for c in names}}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--kernel", default="mfma",
                    help="mfma | mfma_raw (C entry, arguments prepared once) | valu | splitk | "
                         "splitk_atomic | mfma_cfgN | mfma_x<0|1>g<G> "
                         "(forced workgroup order) | streamk_c<config>_g<grid> (forced "
                         "stream-K); mfma and splitk take a suffix _nt, _tn or _tt for "
                         "operands stored transposed")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds for the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--reduce-only", action="store_true",
                    help="only time the array sum on its largest workload (for profiling)")
    ap.add_argument("--valu-calibration", action="store_true",
                    help="only time the FP32 FMA issue-rate probes (the VALU kernel's bound)")
    ap.add_argument("--combine-only", action="store_true",
                    help="only time the split-K combine kernel alone (for profiling)")
    ap.add_argument("--cold-only", action="store_true",
                    help="only time single 2048^3 calls with the caches flushed between them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print duration statistics from a rocprofv3 kernel_trace.csv")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="print counter means from a rocprofv3 counter_collection.csv")
    ap.add_argument("--match", default="sgemm_mfma_kernel")
    ap.add_argument("--last", type=int, default=0, help="use the last N dispatches (0: all)")
    ap.add_argument("--flop", type=float, default=None, help="FLOP per dispatch (summaries)")
    ap.add_argument("--bytes", type=float, default=None, help="bytes per dispatch (summaries)")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.match, args.last,
                                         args.flop, args.bytes), indent=1))
        return 0
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters, args.match, args.last),
                         indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library and this benchmark "
              "run on one GPU (one MI355X); multi-GPU runs are out of scope.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "launches": 5}), flush=True)
        return 0

    if args.valu_calibration:
        print(json.dumps({"valu_calibration": valu_calibration()}), flush=True)
        return 0

    if args.reduce_only:
        print(json.dumps({"reduce": reduce_secondary()}), flush=True)
        return 0
    if args.combine_only:
        print(json.dumps({"combine": combine_secondary()}), flush=True)
        return 0
    if args.cold_only:
        print(json.dumps({"cold": cold_secondary()}), flush=True)
        return 0

    import synth
    from hpc_tiling_amd import perfmodel as pm

    w = synth.workload(args.workload)
    kind = args.kernel
    print(f"[bench] {kind} {w.name}: generating operands", file=sys.stderr, flush=True)
    host, dev, step = setup(w, kind)
    print(f"[bench] warmup {args.warmup}, timing {args.trials} x {args.steps} steps",
          file=sys.stderr, flush=True)
    import hpc_tiling_amd as hta
    probes = (hta.ClockProbe(), hta.ClockProbe())
    # Launch the probe once now: its kernel is loaded on first use, and that
    # host-side pause right before the timed steps would leave the GPU idle for
    # milliseconds -- after such a pause the next ~100 ms of GEMM calls run up
    # to 20 % slower on MI355X although the core clock reads normal.
    for p in probes:
        p.launch()
    extra_warmup = warm(step, args.warmup)
    secs, _ = time_trials(step, args.steps, args.trials, probes)
    sclk_before, sclk_after = (clock_summary(p.mhz()) for p in probes)
    mclk, mclk_err = mclk_mhz()
    trials = trial_stats(secs, args.steps, w.flops)
    ms = trials["ms_per_step_median"]
    value = trials["tflops_median"]

    dominant = {"mfma": "sgemm_mfma_kernel", "valu": "sgemm_valu_kernel",
                "splitk": "sgemm_mfma_kernel (split-K partials)"}.get(kind, "sgemm_mfma_kernel")
    valu = kind == "valu"
    roof = {
        "bound": "alu" if valu else "mfma",
        "kernel": dominant,
        "achieved": value,
        "peak": (pm.PEAK_FP32_VALU if valu else pm.PEAK_FP32_MFMA) / 1e12,
        "unit": "TFLOP/s",
        "frac": None,
        "traffic": read_traffic(kind, w.name),
        "algorithmic_flop_per_launch": w.flops,
        "avg_launch_ms": ms,
        "timing": "HIP events on the launch stream; median of the timed trials",
    }
    if valu:
        roof["peak_note"] = pm.PEAK_FP32_VALU_NOTE
    roof["frac"] = roof["achieved"] / roof["peak"]

    clock_rec = {"sclk_source": ("mi_clock_probe: shader-cycle over reference-counter advance "
                                 "on each of the 8 XCDs, launched on the timing stream right "
                                 "before the first and right after the last timed step"),
                 "sclk_before": sclk_before, "sclk_after": sclk_after,
                 "mclk_source": "amdsmi gpu_metrics current_uclk", "mclk_mhz": mclk}
    if mclk_err:
        clock_rec["mclk_unavailable"] = mclk_err
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_extra_steps": extra_warmup,   # untimed, until 0.2 s of load settles the clock
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded uniform[-1,1) float32 operands, resident in HBM)",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k, "lda": w.lda, "ldb": w.ldb,
                   "ldc": w.ldc, "alpha": w.alpha, "beta": w.beta, "kernel": kind,
                   "layout": "row-major"},
        "frac_of_fp32_peak": value * 1e12 / pm.PEAK_FP32_MFMA,
        "trials": trials,
        "sclk_mhz_before": sclk_before["mean"],
        "sclk_mhz_after": sclk_after["mean"],
        "mclk_mhz": mclk,
        "clocks": clock_rec,
        "roofline": roof,
    }
    del dev, step
    torch.cuda.empty_cache()

    if not args.no_secondary:
        print("[bench] secondary workloads", file=sys.stderr, flush=True)
        pairs = [("mfma", "sgemm_8192x8192x8192_ab"), ("mfma", "sgemm_tails_3001x4997x1023"),
                 ("splitk", "sgemm_tails_3001x4997x1023"),
                 ("splitk", "sgemm_splitk_512x512x262144"),
                 ("splitk_atomic", "sgemm_splitk_512x512x262144"), ("valu", "sgemm_2048x2048x2048"),
                 ("mfma", "sgemm_256x256x256"), ("mfma_raw", "sgemm_256x256x256"),
                 ("mfma_nt", "sgemm_2048x2048x2048"), ("mfma_tn", "sgemm_2048x2048x2048"),
                 ("mfma_tt", "sgemm_2048x2048x2048"), ("mfma_tt", "sgemm_8192x8192x8192_ab"),
                 ("splitk_tn", "sgemm_splitk_512x512x262144"),
                 ("mfma", "sgemm_1536x1536x4096"), ("splitk", "sgemm_1536x1536x4096"),
                 ("mfma", "sgemm_1536x1536x1024"), ("splitk", "sgemm_1536x1536x1024")]
        line["secondary"] = secondary(pairs)
        line["secondary"].append(combine_secondary())
        line["secondary"].append(reduce_secondary())
        line["secondary"].append(cold_secondary())

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        if any(kind.endswith(sfx) for sfx in TRANS_SUFFIXES):
            host = synth.operands(w)   # the oracle leg reads the as-given layout
        line["cpu_baseline"] = cpu_baseline(w, host, args.cpu_budget)
    else:
        line["cpu_baseline"] = None

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

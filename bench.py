#!/usr/bin/env python3
"""SGEMM benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--kernel KIND]

One step is one call of the hot path (C = alpha*A*B + beta*C through the C
ABI) on seeded synthetic operands already resident in HBM.  W untimed steps,
then exactly K steps timed with HIP events on the stream the kernels run on.
Prints ONE JSON line: throughput in TFLOP/s (2mnk per step), the roofline
object of the GEMM kernel (which is the only kernel a step launches for the
default workload, so its average duration is the step time), the CPU oracle
timed on a bounded sample of the same workload, and secondary measurements
of the other workloads.

Only the CPU-baseline leg imports the oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
    torch.cuda.synchronize()
    return (A, B, C), (Ad, Bd, Cd), make_step(kind, w, Av, Bv, Cd[:, :w.n], ws)


SETTLE_S = 0.2
LAST_EXTRA_WARMUP = [0]


def time_steps(step, steps, warmup, settle_s=SETTLE_S):
    """Seconds for exactly `steps` calls after `warmup` untimed ones, measured
    with events on the current stream (the stream the kernels are launched on).
    After an idle spell the GPU clock needs about 30 ms of load to reach its
    steady value, so the untimed warmup continues (in batches of 10 calls,
    counted in LAST_EXTRA_WARMUP) until at least `settle_s` seconds of
    back-to-back calls have run."""
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
    LAST_EXTRA_WARMUP[0] = extra
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3


def cpu_baseline(w, host, budget_s):
    """The oracle on whole output rows of the same workload, as many rows as
    fit the time budget (estimated from a first small batch)."""
    import numpy as np
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


def secondary(kinds_workloads, seconds=0.25):
    """TFLOP/s of other (kernel, workload) pairs, each timed over about
    `seconds` of back-to-back calls after a short warmup."""
    import torch
    import synth
    from hpc_tiling_amd import perfmodel as pm
    out = []
    for kind, name in kinds_workloads:
        w = synth.workload(name)
        host, dev, step = setup(w, kind)
        probe = time_steps(step, 2, warmup=2) / 2
        n = max(3, min(2000, int(seconds / max(probe, 1e-6))))
        dt = time_steps(step, n, warmup=5)
        tf = pm.tflops(w.m, w.n, w.k, dt, reps=n)
        out.append({"workload": name, "kernel": kind, "ms_per_call": 1e3 * dt / n,
                    "tflops": tf, "frac_of_fp32_peak": tf * 1e12 / pm.PEAK_FP32_MFMA})
        del host, dev, step
        torch.cuda.empty_cache()
    return out


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
    probe = time_steps(step, 2, warmup=2) / 2
    n = max(3, min(5000, int(seconds / max(probe, 1e-6))))
    dt = time_steps(step, n, warmup=5) / n
    gbs = 4.0 * x.numel() / dt / 1e9
    res = {"workload": name, "kernel": "reduce_sum", "us_per_call": 1e6 * dt, "gb_per_s": gbs,
           "frac_of_hbm_peak": gbs * 1e9 / pm.PEAK_HBM_BYTES}
    del x, ws
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--kernel", default="mfma",
                    help="mfma | valu | splitk | splitk_atomic | mfma_cfgN; mfma and splitk "
                         "take a suffix _nt, _tn or _tt for operands stored transposed")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds for the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--reduce-only", action="store_true",
                    help="only time the array sum on its largest workload (for profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args(argv)

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

    if args.reduce_only:
        print(json.dumps({"reduce": reduce_secondary()}), flush=True)
        return 0

    import synth
    from hpc_tiling_amd import perfmodel as pm

    w = synth.workload(args.workload)
    kind = args.kernel
    print(f"[bench] {kind} {w.name}: generating operands", file=sys.stderr, flush=True)
    host, dev, step = setup(w, kind)
    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    dt = time_steps(step, args.steps, args.warmup)
    extra_warmup = LAST_EXTRA_WARMUP[0]
    ms = 1e3 * dt / args.steps
    value = pm.tflops(w.m, w.n, w.k, dt, reps=args.steps)

    dominant = {"mfma": "sgemm_mfma_kernel", "valu": "sgemm_valu_kernel",
                "splitk": "sgemm_mfma_kernel (split-K partials)"}.get(kind, "sgemm_mfma_kernel")
    roof = {
        "bound": "mfma" if kind != "valu" else "alu",
        "kernel": dominant,
        "achieved": value,
        "peak": (pm.PEAK_FP32_MFMA if kind != "valu" else pm.PEAK_FP32_VECTOR) / 1e12,
        "unit": "TFLOP/s",
        "frac": None,
        "traffic": read_traffic(kind, w.name),
        "algorithmic_flop_per_launch": w.flops,
        "avg_launch_ms": ms,
        "timing": "HIP events on the launch stream over the timed steps",
    }
    roof["frac"] = roof["achieved"] / roof["peak"]

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
        "roofline": roof,
    }
    del dev, step
    torch.cuda.empty_cache()

    if not args.no_secondary:
        print("[bench] secondary workloads", file=sys.stderr, flush=True)
        pairs = [("mfma", "sgemm_8192x8192x8192_ab"), ("mfma", "sgemm_tails_3001x4997x1023"),
                 ("splitk", "sgemm_splitk_512x512x262144"),
                 ("splitk_atomic", "sgemm_splitk_512x512x262144"), ("valu", "sgemm_2048x2048x2048"),
                 ("mfma", "sgemm_256x256x256"),
                 ("mfma_nt", "sgemm_2048x2048x2048"), ("mfma_tn", "sgemm_2048x2048x2048"),
                 ("mfma_tt", "sgemm_2048x2048x2048"), ("mfma_tt", "sgemm_8192x8192x8192_ab"),
                 ("splitk_tn", "sgemm_splitk_512x512x262144"),
                 ("mfma", "sgemm_1536x1536x4096"), ("splitk", "sgemm_1536x1536x4096"),
                 ("mfma", "sgemm_1536x1536x1024"), ("splitk", "sgemm_1536x1536x1024")]
        line["secondary"] = secondary(pairs)
        line["secondary"].append(reduce_secondary())

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

"""GPU parity of the stream-K schedule (mi_sgemm_streamk, and mi_sgemm_splitk
when its plan chooses it) against the CPU oracle.

Grids are forced across the interesting regimes: one workgroup's worth
(every tile whole, no fixup), grids that divide the tiles (likewise), fewer
workgroups than tiles (whole-tile workgroups first, then the last one to two
rounds' worth of tiles shared), about as many as tiles, and more than tiles
(tiles shared by three or more workgroups); every tile configuration,
transposes, k tails, beta != 0.  Integer-valued operands must be bit-exact; float operands within
the tolerance of tests/parity.py; the schedule is deterministic.
"""
import numpy as np
import pytest

import synth
from parity import assert_close, assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
    N_CFG = hta.mi_sgemm_config_count(hta.KERNEL_MFMA)
else:
    hta = None
    N_CFG = 10


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_sk(w, ta, tb, integer, grid, config, orc):
    A, lda, B, ldb, C = synth.operands_ex(w, ta, tb, integer_twin=integer)
    say("streamk", w.name, w.m, w.n, w.k, ta, tb, "int" if integer else "float", "grid", grid, "cfg", config)
    Ad = torch.from_numpy(A).cuda()
    Bd = torch.from_numpy(B).cuda()
    Cd = torch.from_numpy(C).cuda()
    Av = Ad[:, :w.m].t() if ta else Ad[:, :w.k]
    Bv = Bd[:, :w.k].t() if tb else Bd[:, :w.n]
    hta.sgemm_streamk(Av, Bv, Cd[:, :w.n], w.alpha, w.beta, grid=grid, config=config)
    torch.cuda.synchronize()
    out = Cd.cpu().numpy()
    assert np.array_equal(out[:, w.n:], C[:, w.n:]), "C padding written"
    ref = orc.sgemm(w.m, w.n, w.k, w.alpha, A, lda, B, ldb, w.beta, C, w.ldc, want_g=True,
                    trans_a=bool(ta), trans_b=bool(tb))
    want = ref["C"].reshape(w.m, w.ldc)[:, :w.n]
    what = f"streamk {w.m}x{w.n}x{w.k} ta={ta} tb={tb} grid={grid} cfg={config}"
    if integer:
        assert_exact(out[:, :w.n], want, what)
    else:
        assert_close(out[:, :w.n], want, ref["G"], w.alpha, w.beta, C[:, :w.n], what)
    return out


SHAPES = [(130, 257, 300), (255, 129, 1000), (64, 64, 2049), (300, 200, 33), (1, 1, 5)]
GRIDS = [1, 2, 5, 37, 0, 300]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_streamk_grids(orc, shape, grid):
    m, n, k = shape
    w = synth.Workload(6, "sk", m, n, k, k + 4, n + 4, n + 3, "uniform", "int3", 1.5, 0.5)
    run_sk(w, 0, 0, True, grid, 6, orc)
    run_sk(w.scaled(dist_c="uniform", alpha=1.0, beta=0.0), 0, 0, False, grid, 9, orc)


@pytest.mark.parametrize("config", range(N_CFG))
def test_streamk_every_config(orc, config):
    w = synth.Workload(7, "skcfg", 333, 444, 555, 556, 448, 447, "uniform", "int3", 1.0, -1.0)
    run_sk(w, 0, 0, True, 17, config, orc)
    run_sk(w, 1, 1, True, 0, config, orc)


# 1000 x 1000 has 256 tiles of 64 x 64 and 64 of 128 x 128: grids below half
# the tile count run whole-tile rounds first and share only the last one to
# two rounds' worth of tiles; grid 64 (128 x 128) and 128 (64 x 64) divide
# the tiles and run whole tiles only.
ROUND_CASES = [(6, 37), (6, 100), (6, 128), (9, 7), (9, 29), (9, 64)]


@pytest.mark.parametrize("case", ROUND_CASES, ids=[f"cfg{c}-grid{g}" for c, g in ROUND_CASES])
def test_streamk_whole_tile_rounds(orc, case):
    config, grid = case
    w = synth.Workload(8, "skrounds", 1000, 1000, 300, 304, 1001, 1002, "uniform", "int3", 1.0, 0.5)
    run_sk(w, 0, 0, True, grid, config, orc)
    run_sk(w, 1, 0, True, grid, config, orc)


@pytest.mark.parametrize("combo", [(0, 1), (1, 0), (1, 1)], ids=["NT", "TN", "TT"])
def test_streamk_transposed_and_unaligned(orc, combo):
    ta, tb = combo
    w = synth.Workload(8, "skt", 517, 389, 777, 779, 391, 390, "normal", "normal", 0.75, 2.0)
    run_sk(w, ta, tb, False, 0, -1, orc)
    run_sk(w, ta, tb, True, 23, 0, orc)


def test_streamk_deterministic_and_auto_plan(orc):
    """The automatic split plan takes stream-K at 1536 x 1536 x 4096; two
    runs give the same bits, within the tolerance of the oracle."""
    m = n = 1536
    k = 4096
    plan = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, m, n, k, 0)
    say("streamk auto plan", plan["config"], plan["stream_k_grid"])
    assert plan["stream_k_grid"] > 0
    w = synth.Workload(9, "skauto", m, n, k, k, n, n, "uniform", None, 1.0, 0.0)
    A, B, C = synth.operands(w)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C1 = torch.empty((m, n), device="cuda")
    C2 = torch.empty((m, n), device="cuda")
    ws = hta.splitk_workspace(m, n, k, 0)
    hta.sgemm_splitk(Ad, Bd, C1, splits=0, workspace=ws)
    hta.sgemm_splitk(Ad, Bd, C2, splits=0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    rows = synth.sample_rows([9, 1], m, 24)
    ref = orc.sgemm(m, n, k, 1.0, A, k, B, n, 0.0, C, n, rows=rows, want_g=True)
    assert_close(C1.cpu().numpy()[rows], ref["C"].reshape(m, n)[rows], ref["G"], 1.0, 0.0, 0.0,
                 "auto stream-K")


# Segments that start and stop at every offset of the k loop: a small grid
# cuts tiles at many (tile, k step) positions, and k runs over whole and
# partial last steps.
@pytest.mark.parametrize("config", [6, 9, 12])
def test_streamk_k_sweep(orc, config):
    bk = hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, config, 64, 64, 64, 0)["tile_k"]
    for k in sorted({j * bk + r for j in (1, 2, 3, 5, 8) for r in (0, 1, bk - 1)}):
        w = synth.Workload(10, "skk", 150, 140, k, k + 4, 144, 141, "uniform", "int3", 1.0, 0.5)
        for grid in (3, 7):
            run_sk(w, 0, 0, True, grid, config, orc)


# The fixup writes C in 16-byte groups only when C is 16-byte aligned and ldc
# is a multiple of 4.  A C that starts 1-3 floats past an aligned address
# (ldc 132, a multiple of 4) must take the element-wise stores, as must
# ldc 133; column 128 of n = 129 is a partial group at the right edge.
# Grid 37 over 4 tiles of 10 k steps shares every tile among 9-10
# workgroups, so the fixup adds parts in several groups of loads.
@pytest.mark.parametrize("off", [0, 1, 2, 3])
@pytest.mark.parametrize("ldc", [132, 133])
def test_streamk_c_alignment(orc, off, ldc):
    w = synth.Workload(11, "skalign", 130, 129, 300, 304, 132, ldc, "uniform", "int3", 1.0, 0.5)
    A, lda, B, ldb, C = synth.operands_ex(w, 0, 0, integer_twin=True)
    say("streamk C offset", off, "ldc", ldc)
    flat = torch.full((off + C.size + 8,), float("nan"), device="cuda")
    flat[off:off + C.size] = torch.from_numpy(C.reshape(-1)).cuda()
    Cv = torch.as_strided(flat, (w.m, w.n), (ldc, 1), off)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    hta.sgemm_streamk(Ad[:, :w.k], Bd[:, :w.n], Cv, w.alpha, w.beta, grid=37, config=9)
    torch.cuda.synchronize()
    got = flat.cpu().numpy()
    assert np.isnan(got[:off]).all() and np.isnan(got[off + C.size:]).all(), "wrote outside C"
    out = got[off:off + C.size].reshape(w.m, ldc)
    assert np.array_equal(out[:, w.n:], C[:, w.n:]), "C padding written"
    ref = orc.sgemm(w.m, w.n, w.k, w.alpha, A, lda, B, ldb, w.beta, C, ldc)
    assert_exact(out[:, :w.n], ref["C"].reshape(w.m, ldc)[:, :w.n],
                 f"streamk C offset {off} ldc {ldc}")


@pytest.mark.parametrize("shape", [(768, 768, 1024), (1536, 1536, 1024)],
                         ids=["768x768x1024", "1536x1536x1024"])
def test_streamk_auto_one_per_cu(orc, shape):
    """Small grids with 1024 <= k <= 2048: the automatic split plan runs the
    64 x 64 x 32 tile on stream-K with one workgroup per CU.  Integer operands
    and beta != 0: bit-exact against the oracle on every element."""
    m, n, k = shape
    plan = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, m, n, k, 0)
    assert (plan["config"], plan["stream_k_grid"]) == (6, 256)
    w = synth.Workload(12, "skone", m, n, k, k, n, n, "uniform", "int3", 1.0, 0.5)
    A, B, C = synth.operands(w, integer_twin=True)
    say("streamk auto one per CU", m, n, k)
    Ad, Bd, Cd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), torch.from_numpy(C).cuda()
    hta.sgemm_splitk(Ad, Bd, Cd, alpha=1.0, beta=0.5, splits=0)
    torch.cuda.synchronize()
    ref = orc.sgemm(m, n, k, 1.0, A, k, B, n, 0.5, C, n)
    assert_exact(Cd.cpu().numpy(), ref["C"].reshape(m, n), f"stream-K one per CU {m}x{n}x{k}")
    # float operands: the parts are added in a fixed order, so two runs agree bitwise
    Af, Bf, _ = synth.operands(w)
    Afd, Bfd = torch.from_numpy(Af).cuda(), torch.from_numpy(Bf).cuda()
    C1 = hta.sgemm_splitk(Afd, Bfd, splits=0)
    C2 = hta.sgemm_splitk(Afd, Bfd, splits=0)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


# The one-per-CU route on float operands, at and next to the ends of its k
# range (the rule takes 1024 <= k <= 2048), with beta != 0 and one operand
# stored transposed: every element within the tolerance of the oracle, and
# the planner's choice asserted on each side of both ends.
ONE_PER_CU_CASES = [(768, 768, k, ta) for k in (1023, 1024, 1025) for ta in (0, 1)] + \
                   [(1536, 1536, k, ta) for k in (2047, 2048, 2049) for ta in (0, 1)]


@pytest.mark.parametrize("case", ONE_PER_CU_CASES,
                         ids=[f"{m}x{n}x{k}{'_tn' if ta else ''}" for m, n, k, ta in ONE_PER_CU_CASES])
def test_streamk_one_per_cu_float_boundaries(orc, case):
    m, n, k, ta = case
    plan = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, m, n, k, 0)
    one_per_cu = (plan["config"], plan["stream_k_grid"]) == (6, 256)
    assert one_per_cu == (1024 <= k <= 2048), plan
    w = synth.Workload(13, "skonef", m, n, k, k + 4, n + 4, n + 3, "uniform", "normal", 1.25, 0.5)
    A, lda, B, ldb, C = synth.operands_ex(w, ta, 0)
    say("one per CU float", m, n, k, "ta", ta, "plan", plan["config"], plan["stream_k_grid"])
    Ad, Bd, Cd = (torch.from_numpy(x).cuda() for x in (A, B, C))
    Av = Ad[:, :m].t() if ta else Ad[:, :k]
    hta.sgemm_splitk(Av, Bd[:, :n], Cd[:, :n], w.alpha, w.beta, splits=0)
    torch.cuda.synchronize()
    out = Cd.cpu().numpy()
    assert np.array_equal(out[:, n:], C[:, n:]), "C padding written"
    ref = orc.sgemm(m, n, k, w.alpha, A, lda, B, ldb, w.beta, C, w.ldc, want_g=True,
                    trans_a=bool(ta))
    assert_close(out[:, :n], ref["C"].reshape(m, w.ldc)[:, :n], ref["G"], w.alpha, w.beta,
                 C[:, :n], f"one per CU {m}x{n}x{k} ta={ta}")

"""GPU parity of the transposed-operand forms (mi_sgemm_ex, mi_sgemm_splitk_ex
and the forced-configuration entry points with trans flags) against the CPU
oracle, which reads the same stored arrays with the same flags.

Besides the tolerance and integer-exact bars of tests/parity.py: a transposed
operand is staged into LDS in its own layout but feeds the matrix cores the
same values in the same order as the as-given layout, so for one tile
configuration the result of every storage order is bitwise the result of the
as-given call.
"""
import numpy as np
import pytest

import synth
from parity import assert_close, assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
    N_MFMA_CFG = hta.mi_sgemm_config_count(hta.KERNEL_MFMA)
else:  # collected on a CPU host: every test here is skipped below
    hta = None
    N_MFMA_CFG = 10

COMBOS = [(0, 1), (1, 0), (1, 1)]
COMBO_IDS = ["NT", "TN", "TT"]


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def logical_view(arr, width, trans):
    """Device copy of a stored (padded) array and the logical operand view:
    the stored block itself, or its transpose (a column-major view)."""
    t = torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")
    v = t[:, :width]
    return t, (v.t() if trans else v)


def run_kind(kind, A, B, C, alpha, beta):
    if kind == "mfma":
        hta.sgemm(A, B, C, alpha, beta)
    elif kind.startswith("mfma_cfg"):
        hta.sgemm(A, B, C, alpha, beta, config=int(kind[len("mfma_cfg"):]))
    elif kind == "splitk":
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=0)
    elif kind.startswith("splitk_cfg"):
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=min(5, A.shape[1]),
                         config=int(kind[len("splitk_cfg"):]))
    elif kind.startswith("splitk"):
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=min(int(kind[len("splitk"):]), A.shape[1]))
    else:
        raise ValueError(kind)
    torch.cuda.synchronize()


def gpu_gemm_ex(kind, w, ta, tb, A, B, C):
    Ad, Av = logical_view(A, w.m if ta else w.k, ta)
    Bd, Bv = logical_view(B, w.k if tb else w.n, tb)
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to("cuda")
    run_kind(kind, Av, Bv, Cd[:, :w.n], w.alpha, w.beta)
    out = Cd.cpu().numpy()
    del Ad, Bd, Cd
    return out


def check(orc, kind, w, ta, tb, integer, rows=None):
    A, lda, B, ldb, C = synth.operands_ex(w, ta, tb, integer_twin=integer)
    say(kind, w.name, "T" if ta else "N", "T" if tb else "N", "int" if integer else "float",
        f"lda={lda} ldb={ldb}")
    out = gpu_gemm_ex(kind, w, ta, tb, A, B, C)
    assert np.array_equal(out[:, w.n:], C[:, w.n:]), "C padding written"
    assert np.all(np.isfinite(out[:, :w.n])), "non-finite output (NaN pad read?)"
    ref = orc.sgemm(w.m, w.n, w.k, w.alpha, A, lda, B, ldb, w.beta, C, w.ldc,
                    rows=rows, want_g=True, trans_a=bool(ta), trans_b=bool(tb))
    sel = slice(None) if rows is None else rows
    want = ref["C"].reshape(w.m, w.ldc)[sel, :w.n]
    got = out[sel, :w.n]
    what = f"{kind} {w.name} ta={ta} tb={tb}"
    if integer:
        assert_exact(got, want, what + " int")
    else:
        assert_close(got, want, ref["G"], w.alpha, w.beta, C[sel, :w.n], what)
    return out


# ---------------------------------------------------------------------------
# Small ragged shapes, every tile configuration, 16-byte and 4-byte loads
# ---------------------------------------------------------------------------
KINDS = (["mfma", "splitk", "splitk3"] + [f"mfma_cfg{i}" for i in range(N_MFMA_CFG)]
         + [f"splitk_cfg{i}" for i in range(N_MFMA_CFG)])
SHAPES = [(1, 1, 1), (7, 9, 5), (33, 65, 17), (130, 257, 300), (255, 129, 64), (64, 128, 2049)]


@pytest.mark.parametrize("ld_pad", [0, 3], ids=["ld=w", "ld=w+3"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("combo", COMBOS, ids=COMBO_IDS)
@pytest.mark.parametrize("kind", KINDS)
def test_small_shapes_transposed(orc, kind, combo, shape, ld_pad):
    m, n, k = shape
    ta, tb = combo
    w = synth.Workload(0, "small", m, n, k, k + ld_pad, n + ld_pad, n + ld_pad + 1,
                       "uniform", None, 1.0, 0.0)
    check(orc, kind, w, ta, tb, integer=False)
    check(orc, kind, w.scaled(dist_c="int3", alpha=1.5, beta=0.5), ta, tb, integer=True)


@pytest.mark.parametrize("config", range(N_MFMA_CFG))
def test_transposed_bitwise_equals_as_given(config):
    """Same tile configuration, same values: every storage order gives the
    bits of the as-given call (full-k and split-K kernels)."""
    w = synth.Workload(5, "bitwise", 301, 259, 777, 780, 260, 263, "normal", "normal", 1.25, -0.5)
    A, B, C = synth.operands(w)
    say("bitwise", config)
    base = {}
    for kind in (f"mfma_cfg{config}", f"splitk_cfg{config}"):
        Ad, Av = logical_view(A, w.k, False)
        Bd, Bv = logical_view(B, w.n, False)
        Cd = torch.from_numpy(C).to("cuda")
        run_kind(kind, Av, Bv, Cd[:, :w.n], w.alpha, w.beta)
        base[kind] = Cd.cpu().numpy()
    for ta, tb in COMBOS:
        At, lda, Bt, ldb, _ = synth.operands_ex(w, ta, tb)
        for kind in base:
            out = gpu_gemm_ex(kind, w, ta, tb, At, Bt, C)
            assert_exact(out, base[kind], f"{kind} ta={ta} tb={tb} lda={lda} ldb={ldb}")


# ---------------------------------------------------------------------------
# Workload sizes
# ---------------------------------------------------------------------------
# The as-given GPU result of one (kind, workload, twin), kept while the three
# transposed forms of it are checked.
_AS_GIVEN = {}


def as_given(kind, w, integer):
    key = (kind, w, integer)
    if key not in _AS_GIVEN:
        _AS_GIVEN.clear()
        A, B, C = synth.operands(w, integer_twin=integer)
        say(kind, w.name, "as given", "int" if integer else "float")
        _AS_GIVEN[key] = gpu_gemm_ex(kind, w, 0, 0, A, B, C)
    return _AS_GIVEN[key]


def workload_check(orc, kind, w, combo, integer, nrows):
    """Sampled rows against the oracle (its transposed-operand walk is
    strided, so whole products at these sizes are slow), and every element
    bitwise against the as-given call: the same tile configuration and plan
    feed the matrix cores the same values in the same order."""
    out = check(orc, kind, w, *combo, integer, rows=synth.sample_rows([w.wid, 98], w.m, nrows))
    assert_exact(out, as_given(kind, w, integer), f"{kind} {w.name} ta,tb={combo} vs as given")


@pytest.mark.parametrize("combo", COMBOS, ids=COMBO_IDS)
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_2048_transposed(orc, combo, integer):
    workload_check(orc, "mfma", synth.workload(1), combo, integer, 48)


@pytest.mark.parametrize("combo", COMBOS, ids=COMBO_IDS)
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_8192_transposed(orc, combo, integer):
    workload_check(orc, "mfma", synth.workload(2), combo, integer, 8)


@pytest.mark.parametrize("combo", COMBOS, ids=COMBO_IDS)
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_tails_transposed(orc, combo, integer):
    workload_check(orc, "mfma", synth.workload(3), combo, integer, 32)


@pytest.mark.parametrize("combo", COMBOS, ids=COMBO_IDS)
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_splitk_transposed(orc, combo, integer):
    workload_check(orc, "splitk", synth.workload(4), combo, integer, 4)


# ---------------------------------------------------------------------------
# Interface cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["mfma", "splitk"])
def test_misaligned_transposed(kind):
    """Transposed operands one float off 16-byte alignment (4-byte loads)."""
    say("misaligned transposed", kind)
    m, n, k = 97, 131, 203
    rng = np.random.default_rng(7)
    Ai = rng.integers(-3, 4, (m, k)).astype(np.float32)
    Bi = rng.integers(-3, 4, (k, n)).astype(np.float32)
    want = (Ai.astype(np.int64) @ Bi.astype(np.int64)).astype(np.float32)
    # stored transposes with one leading column, so the logical blocks start at
    # an odd float offset
    At = torch.from_numpy(np.concatenate([np.zeros((k, 1), np.float32), Ai.T], axis=1)).cuda()
    Bt = torch.from_numpy(np.concatenate([np.zeros((n, 1), np.float32), Bi.T], axis=1)).cuda()
    C = torch.zeros((m, n), device="cuda")
    run_kind(kind, At[:, 1:].t(), Bt[:, 1:].t(), C, 1.0, 0.0)
    assert_exact(C.cpu().numpy(), want, "misaligned transposed")


def test_column_major_c():
    """A column-major C is computed as the row-major C^T = op(B)^T op(A)^T."""
    say("column-major C")
    m, n, k = 150, 70, 90
    rng = np.random.default_rng(11)
    Ai = rng.integers(-3, 4, (m, k)).astype(np.float32)
    Bi = rng.integers(-3, 4, (k, n)).astype(np.float32)
    Ci = rng.integers(-3, 4, (m, n)).astype(np.float32)
    want = ((3 * (Ai.astype(np.int64) @ Bi.astype(np.int64)) + Ci) / 2).astype(np.float32)
    for ta, tb in [(0, 0)] + COMBOS:
        A = torch.from_numpy(np.ascontiguousarray(Ai.T)).cuda().t() if ta else torch.from_numpy(Ai).cuda()
        B = torch.from_numpy(np.ascontiguousarray(Bi.T)).cuda().t() if tb else torch.from_numpy(Bi).cuda()
        Cs = torch.from_numpy(np.ascontiguousarray(Ci.T)).cuda()   # n x m storage
        hta.sgemm(A, B, Cs.t(), 1.5, 0.5)
        torch.cuda.synchronize()
        assert_exact(Cs.t().cpu().numpy(), want, f"column-major C ta={ta} tb={tb}")

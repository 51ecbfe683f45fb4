"""GPU checks of the split-K combine on its own (mi_sgemm_splitk_combine):
C <- alpha * sum_s parts[s] + beta * C.

The expected values are sums written out in float64 with numpy (the
definition of the step: page aerisun.top, section
"先在线程内累加，再交换部分和", adds partial sums; any order is correct up to
rounding).  Integer-valued partials give exact sums in every order, so the
result must match bitwise; float partials must stay within
2e-5 * |alpha| * sum_s |parts[s]| + 1e-6 * |beta * C| + 1e-7, the bar of the
GEMM with sum_s |parts[s]| in place of G.  Slice entries past m * n are
read (whole 16-byte groups) but must not reach C: they hold NaN here.
"""
import numpy as np
import pytest

from parity import assert_close, assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
else:
    hta = None

SENTINEL = np.float32(-12345.5)


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_combine(parts, m, n, ldc, alpha, beta, C):
    """parts: (S, slice) float32 host array; C: (m, ldc) host array."""
    Pd = torch.from_numpy(np.ascontiguousarray(parts)).cuda()
    Cd = torch.from_numpy(np.ascontiguousarray(C)).cuda()
    hta.splitk_combine(Pd, Cd[:, :n], alpha, beta)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


def make(S, m, n, ldc, integer, seed):
    rng = np.random.default_rng([seed, S, m, n])
    mn = m * n
    slice_ = (mn + 3) // 4 * 4 + 4 * (seed % 3)
    parts = np.full((S, slice_), np.nan, np.float32)
    if integer:
        parts[:, :mn] = rng.integers(-3, 4, (S, mn)).astype(np.float32)
        Cl = rng.integers(-3, 4, (m, n)).astype(np.float32)
    else:
        parts[:, :mn] = (rng.random((S, mn), dtype=np.float32) * 2 - 1)
        Cl = rng.standard_normal((m, n)).astype(np.float32)
    C = np.full((m, ldc), SENTINEL, np.float32)
    C[:, :n] = Cl
    return parts, C


SHAPES = [(1, 1), (1, 3), (7, 9), (13, 5), (100, 257), (512, 512)]
SPLITS = [1, 2, 3, 4, 5, 7, 16, 37, 64]


@pytest.mark.parametrize("S", SPLITS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}" for m, n in SHAPES])
def test_combine_integer_exact(shape, S):
    m, n = shape
    ldc = n + 3
    parts, C = make(S, m, n, ldc, True, 1)
    say("combine int", m, n, S)
    out = run_combine(parts, m, n, ldc, 1.5, 0.5, C)
    total = parts[:, :m * n].astype(np.int64).sum(axis=0).reshape(m, n)
    want = (1.5 * total + 0.5 * C[:, :n].astype(np.float64)).astype(np.float32)
    assert_exact(out[:, :n], want, f"combine {m}x{n} S={S}")
    assert np.array_equal(out[:, n:], C[:, n:]), "C padding written"


@pytest.mark.parametrize("S", [1, 3, 16, 64])
@pytest.mark.parametrize("beta", [0.0, -0.75], ids=["beta0", "beta"])
def test_combine_float_bound_and_repeat(S, beta):
    m, n, ldc = 300, 517, 520
    parts, C = make(S, m, n, ldc, False, 2)
    if beta == 0.0:
        C[:, :n] = np.nan   # beta == 0: C is written without being read
    say("combine float", m, n, S, beta)
    out = run_combine(parts, m, n, ldc, 0.5, beta, C)
    out2 = run_combine(parts, m, n, ldc, 0.5, beta, C)
    assert np.array_equal(out, out2, equal_nan=True), "combine not bitwise repeatable"
    p = parts[:, :m * n].astype(np.float64)
    want = 0.5 * p.sum(axis=0).reshape(m, n)
    if beta != 0.0:
        want = want + beta * C[:, :n].astype(np.float64)
    G = np.abs(p).sum(axis=0).reshape(m, n)
    assert_close(out[:, :n], want, G, 0.5, beta, C[:, :n], f"combine float S={S}")
    assert np.array_equal(out[:, n:], C[:, n:]), "C padding written"

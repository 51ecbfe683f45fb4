"""GPU parity of the array sum (mi_reduce_sum) against the CPU oracle.

Bar: |gpu - exact| <= D * 2^-24 * sum|x| + 1e-30, with D the kernel's stated
maximum number of additions on any path (mi_reduce_sum_max_additions) and
the exact sum taken from the oracle (double, whose own error is below
n * 2^-53 * sum|x|); integer-valued inputs are exact.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
else:
    hta = None


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_sum(xh, offset=0):
    base = torch.zeros(xh.size + offset, dtype=torch.float32, device="cuda")
    base[offset:] = torch.from_numpy(xh).cuda()
    x = base[offset:]
    out = hta.reduce_sum(x)
    torch.cuda.synchronize()
    return float(out.cpu()[0])


def check(orc, xh, offset=0, what=""):
    print("[case] reduce", what, xh.size, offset, flush=True)
    got = gpu_sum(xh, offset)
    s, a = orc.sum(xh)
    d = hta.mi_reduce_sum_max_additions(xh.size)
    tol = d * 2.0 ** -24 * a + xh.size * 2.0 ** -53 * a + 1e-30
    assert abs(got - s) <= tol, (what, xh.size, got, s, tol)


SIZES = [0, 1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 1023, 4096, 65537, 1 << 20, (1 << 22) + 3]


@pytest.mark.parametrize("n", SIZES)
def test_sum_sizes(orc, n):
    check(orc, synth.vector(n), 0, "uniform")


@pytest.mark.parametrize("n", [1, 5, 1000, 65537, (1 << 22) + 1])
def test_sum_integers_exact(orc, n):
    xh = synth.vector(n, integer_twin=True)
    got = gpu_sum(xh)
    s, _ = orc.sum(xh)
    assert got == s


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_sum_unaligned(orc, offset):
    check(orc, synth.vector(100003), offset, "unaligned")


@pytest.mark.parametrize("name", list(synth.REDUCE_WORKLOADS))
def test_sum_workloads(orc, name):
    check(orc, synth.vector(name), 0, name)
    xi = synth.vector(name, integer_twin=True)
    s, _ = orc.sum(xi)
    assert gpu_sum(xi) == s


def test_sum_deterministic():
    xh = synth.vector(1 << 22)
    assert gpu_sum(xh) == gpu_sum(xh)


def test_sum_cancellation_and_scale(orc):
    xh = np.concatenate([np.full(1000, 1e8, np.float32), np.ones(3000, np.float32),
                         np.full(1000, -1e8, np.float32)])
    check(orc, xh, 0, "cancellation")
    check(orc, np.full(1 << 20, 3.0e-3, np.float32), 0, "constant")

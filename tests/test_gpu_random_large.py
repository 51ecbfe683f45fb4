"""Seeded random products of larger sizes through the automatic entries.

Sizes up to 2500 x 2500 with k up to 20000 (capped at 6e9 multiply-adds),
so that the planner's own choices are exercised: the tile configurations
for short and long grids, split-K slice counts, the stream-K schedules
(among them the one-workgroup-per-CU route for 1024 <= k <= 2048), each with
transposes, padded leading dimensions, an odd base offset (no 16-byte
loads), alpha and beta.  Integer-valued operands must match the oracle bit
for bit, uniform floats within the tolerance of tests/parity.py; the C pads
must stay untouched.
"""
import numpy as np
import pytest

from parity import assert_close, assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from storage import stored_device  # noqa: E402

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
else:
    hta = None

CASES = 200


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", range(CASES))
def test_random_large_configuration(orc, case):
    rng = np.random.default_rng([4242, case])
    m, n = int(rng.integers(1, 2500)), int(rng.integers(1, 2500))
    k = int(rng.choice([rng.integers(1, 4000), rng.integers(1000, 2100), rng.integers(4000, 20000)]))
    if m * n * k > 6e9:
        k = max(1, int(6e9 // (m * n)))
    ta, tb = bool(rng.random() < 0.3), bool(rng.random() < 0.3)
    pads = [int(rng.choice([0, 1, 4, 12])) for _ in range(3)]
    off = int(rng.random() < 0.2)
    integer = bool(rng.random() < 0.5)
    alpha, beta = float(rng.choice([1.0, -0.5, 1.5])), float(rng.choice([0.0, 0.5, 1.0]))
    path = str(rng.choice(["mfma", "splitk", "streamk"]))
    print(f"[case] {case}: {m}x{n}x{k} ta={ta} tb={tb} pads={pads} off={off} int={integer} "
          f"alpha={alpha} beta={beta} path={path}", flush=True)
    if integer:
        Av = rng.integers(-3, 4, (m, k)).astype(np.float32)
        Bv = rng.integers(-3, 4, (k, n)).astype(np.float32)
        Cv = rng.integers(-3, 4, (m, n)).astype(np.float32)
    else:
        Av = 2 * rng.random((m, k), dtype=np.float32) - 1
        Bv = 2 * rng.random((k, n), dtype=np.float32) - 1
        Cv = 2 * rng.random((m, n), dtype=np.float32) - 1
    keep_a, A, lda = stored_device(Av, ta, pads[0], off)
    keep_b, B, ldb = stored_device(Bv, tb, pads[1], off)
    ldc = n + pads[2]
    Cfull = torch.full((m, ldc), -12345.5, device="cuda")
    Cfull[:, :n] = torch.from_numpy(Cv).cuda()
    C = Cfull[:, :n]
    if path == "mfma":
        hta.sgemm(A, B, C, alpha, beta)
    elif path == "splitk":
        hta.sgemm_splitk(A, B, C, alpha, beta)
    else:
        hta.sgemm_streamk(A, B, C, alpha, beta)
    torch.cuda.synchronize()
    out = Cfull.cpu().numpy()
    assert np.all(out[:, n:] == np.float32(-12345.5)), "C padding written"

    # the oracle reads the same storage (transposed or not, same ld)
    Ah = np.ascontiguousarray(Av.T) if ta else Av
    Bh = np.ascontiguousarray(Bv.T) if tb else Bv
    Ah = np.pad(Ah, ((0, 0), (0, lda - Ah.shape[1])), constant_values=np.nan).astype(np.float32)
    Bh = np.pad(Bh, ((0, 0), (0, ldb - Bh.shape[1])), constant_values=np.nan).astype(np.float32)
    Ch = np.pad(Cv, ((0, 0), (0, pads[2])), constant_values=-12345.5).astype(np.float32)
    ref = orc.sgemm(m, n, k, alpha, Ah, lda, Bh, ldb, beta, Ch, ldc, want_g=True,
                    trans_a=ta, trans_b=tb)
    want = ref["C"].reshape(m, ldc)[:, :n]
    if integer:
        assert_exact(out[:, :n], want, f"case {case}")
    else:
        assert_close(out[:, :n], want, ref["G"], alpha, beta, Cv, f"case {case}")

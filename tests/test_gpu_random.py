"""Seeded random configurations against the CPU oracle.

Each case draws sizes (1..700; 1..1100 for the VALU cases), leading-dimension
pads, a one-float base offset (which turns off 16-byte loads), transposes,
alpha / beta (0 included), and an entry point with its tile configuration and
slice count; the
operands are integer-valued (then the result must be bit-exact) or uniform
floats (then within the tolerance of tests/parity.py).  The oracle reads the
same stored arrays with the same flags.
"""
import numpy as np
import pytest

from parity import assert_close, assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from storage import stored_device  # noqa: E402

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
    N_CFG = hta.mi_sgemm_config_count(hta.KERNEL_MFMA)
else:
    hta = None
    N_CFG = 10

CASES = 1000


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", range(CASES))
def test_random_configuration(orc, case):
    rng = np.random.default_rng([777, case])
    m, n, k = (int(v) for v in rng.integers(1, 701, size=3))
    if rng.random() < 0.2:
        k = int(rng.integers(1, 40))                    # short k: one partial step
    ta, tb = bool(rng.random() < 0.4), bool(rng.random() < 0.4)
    pad_a, pad_b, pad_c = (int(rng.choice([0, 1, 3, 4])) for _ in range(3))
    off = int(rng.random() < 0.25)
    integer = bool(rng.random() < 0.5)
    alpha = float(rng.choice([1.0, -0.5, 2.0, 0.0])) if rng.random() < 0.3 else 1.0
    beta = float(rng.choice([0.0, 0.5, 1.0, -1.5]))
    path = str(rng.choice(["mfma", "mfma_cfg", "splitk", "splitk_cfg", "atomic"]))
    cfg = int(rng.integers(0, N_CFG))
    splits = int(rng.integers(1, 9))
    if path == "atomic" and (ta or tb):
        path = "splitk"
    print(f"[case] {case}: {m}x{n}x{k} ta={ta} tb={tb} pads={pad_a},{pad_b},{pad_c} off={off} "
          f"int={integer} alpha={alpha} beta={beta} path={path} cfg={cfg} splits={splits}", flush=True)

    if integer:
        Av = rng.integers(-3, 4, (m, k)).astype(np.float32)
        Bv = rng.integers(-3, 4, (k, n)).astype(np.float32)
        Cv = rng.integers(-3, 4, (m, n)).astype(np.float32)
    else:
        Av = (2 * rng.random((m, k), dtype=np.float32) - 1).astype(np.float32)
        Bv = (2 * rng.random((k, n), dtype=np.float32) - 1).astype(np.float32)
        Cv = (2 * rng.random((m, n), dtype=np.float32) - 1).astype(np.float32)
    keep_a, A, lda = stored_device(Av, ta, pad_a, off)
    keep_b, B, ldb = stored_device(Bv, tb, pad_b, off)
    ldc = n + pad_c
    Cfull = torch.full((m, ldc), -12345.5, device="cuda")
    Cfull[:, :n] = torch.from_numpy(Cv).cuda()
    C = Cfull[:, :n]

    if path == "mfma":
        hta.sgemm(A, B, C, alpha, beta)
    elif path == "mfma_cfg":
        hta.sgemm(A, B, C, alpha, beta, config=cfg)
    elif path == "splitk":
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=min(splits, k) if rng.random() < 0.5 else 0)
    elif path == "splitk_cfg":
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=min(splits, k), config=cfg)
    else:
        hta.sgemm_splitk_atomic(A, B, C, alpha, beta, splits=min(splits, k))
    torch.cuda.synchronize()
    out = Cfull.cpu().numpy()
    assert np.all(out[:, n:] == np.float32(-12345.5)), "C padding written"

    # the oracle reads the same storage (transposed or not, same ld)
    Ah = (np.ascontiguousarray(Av.T) if ta else Av)
    Bh = (np.ascontiguousarray(Bv.T) if tb else Bv)
    Ah = np.pad(Ah, ((0, 0), (0, lda - Ah.shape[1])), constant_values=np.nan).astype(np.float32)
    Bh = np.pad(Bh, ((0, 0), (0, ldb - Bh.shape[1])), constant_values=np.nan).astype(np.float32)
    Ch = np.pad(Cv, ((0, 0), (0, pad_c)), constant_values=-12345.5).astype(np.float32)
    ref = orc.sgemm(m, n, k, alpha, Ah, lda, Bh, ldb, beta, Ch, ldc, want_g=True,
                    trans_a=ta, trans_b=tb)
    want = ref["C"].reshape(m, ldc)[:, :n]
    if integer:
        assert_exact(out[:, :n], want, f"case {case}")
    else:
        assert_close(out[:, :n], want, ref["G"], alpha, beta, Cv, f"case {case}")


VALU_CASES = 200


@pytest.mark.parametrize("case", range(VALU_CASES))
def test_random_valu_configuration(orc, case):
    """The register-tiled VALU kernel (operands as given) on seeded random
    shapes up to 1100 per side: its automatic choice and both forced
    configurations (one k group, two), with and without 16-byte loads."""
    rng = np.random.default_rng([778, case])
    m, n = (int(v) for v in rng.integers(1, 1101, size=2))
    k = int(rng.integers(1, 40)) if rng.random() < 0.2 else int(rng.integers(1, 1101))
    pad_a, pad_b, pad_c = (int(rng.choice([0, 1, 4])) for _ in range(3))
    off = int(rng.random() < 0.2)
    integer = bool(rng.random() < 0.5)
    alpha = float(rng.choice([1.0, -0.5, 2.0])) if rng.random() < 0.3 else 1.0
    beta = float(rng.choice([0.0, 0.5, 1.0, -1.5]))
    config = [None, 0, 1][int(rng.integers(0, 3))]
    print(f"[case] valu {case}: {m}x{n}x{k} pads={pad_a},{pad_b},{pad_c} off={off} "
          f"int={integer} alpha={alpha} beta={beta} config={config}", flush=True)
    if integer:
        Av = rng.integers(-3, 4, (m, k)).astype(np.float32)
        Bv = rng.integers(-3, 4, (k, n)).astype(np.float32)
        Cv = rng.integers(-3, 4, (m, n)).astype(np.float32)
    else:
        Av = (2 * rng.random((m, k), dtype=np.float32) - 1).astype(np.float32)
        Bv = (2 * rng.random((k, n), dtype=np.float32) - 1).astype(np.float32)
        Cv = (2 * rng.random((m, n), dtype=np.float32) - 1).astype(np.float32)
    keep_a, A, lda = stored_device(Av, False, pad_a, off)
    keep_b, B, ldb = stored_device(Bv, False, pad_b, off)
    ldc = n + pad_c
    Cfull = torch.full((m, ldc), -12345.5, device="cuda")
    Cfull[:, :n] = torch.from_numpy(Cv).cuda()
    hta.sgemm_valu(A, B, Cfull[:, :n], alpha, beta, config=config)
    torch.cuda.synchronize()
    out = Cfull.cpu().numpy()
    assert np.all(out[:, n:] == np.float32(-12345.5)), "C padding written"

    Ah = np.pad(Av, ((0, 0), (0, lda - k)), constant_values=np.nan).astype(np.float32)
    Bh = np.pad(Bv, ((0, 0), (0, ldb - n)), constant_values=np.nan).astype(np.float32)
    Ch = np.pad(Cv, ((0, 0), (0, pad_c)), constant_values=-12345.5).astype(np.float32)
    ref = orc.sgemm(m, n, k, alpha, Ah, lda, Bh, ldb, beta, Ch, ldc, want_g=True)
    want = ref["C"].reshape(m, ldc)[:, :n]
    if integer:
        assert_exact(out[:, :n], want, f"valu case {case}")
    else:
        assert_close(out[:, :n], want, ref["G"], alpha, beta, Cv, f"valu case {case}")

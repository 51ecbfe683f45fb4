"""GPU parity: the HIP kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bars: floating-point results within the tolerance in tests/parity.py; results
on integer-valued operands bit-exact; padding of A and B (NaN) never read,
padding of C (sentinel) never written.  Every output element is compared, at
the five workload sizes too: the oracle computes each full-size product once
(float and integer twin) and every path is checked against it.
"""
import numpy as np
import pytest

import synth
from parity import assert_close, assert_close_blocked, assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
    N_MFMA_CFG = hta.mi_sgemm_config_count(hta.KERNEL_MFMA)
else:  # collected on a CPU host: every test here is skipped below
    hta = None
    N_MFMA_CFG = 6


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def upload(arr, cols):
    t = torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")
    return t, t[:, :cols]


def run_kernel(kind, A, B, C, alpha, beta):
    """Launch one of the paths on tensor views; returns after synchronising."""
    if kind == "mfma":
        hta.sgemm(A, B, C, alpha, beta)
    elif kind.startswith("mfma_cfg"):
        hta.sgemm(A, B, C, alpha, beta, config=int(kind[len("mfma_cfg"):]))
    elif kind == "valu":
        hta.sgemm_valu(A, B, C, alpha, beta)
    elif kind.startswith("valu_cfg"):
        hta.sgemm_valu(A, B, C, alpha, beta, config=int(kind[len("valu_cfg"):]))
    elif kind == "splitk":
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=0)
    elif kind.startswith("splitk_atomic"):
        splits = min(int(kind[len("splitk_atomic"):] or 0), A.shape[1])
        hta.sgemm_splitk_atomic(A, B, C, alpha, beta, splits=splits)
    elif kind.startswith("splitk_cfg"):
        # forced partial-kernel tiles with an odd slice count (at most k)
        splits = min(5, A.shape[1])
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=splits, config=int(kind[len("splitk_cfg"):]))
    elif kind.startswith("splitk"):
        # a split count above k is an argument error; ask for at most k slices
        splits = min(int(kind[len("splitk"):]), A.shape[1])
        hta.sgemm_splitk(A, B, C, alpha, beta, splits=splits)
    else:
        raise ValueError(kind)
    torch.cuda.synchronize()


def gpu_gemm(kind, w, A, B, C):
    """Run `kind` on padded host arrays; returns the full padded C back."""
    Ad, Av = upload(A, w.k)
    Bd, Bv = upload(B, w.n)
    Cd, Cv = upload(C, w.n)
    run_kernel(kind, Av, Bv, Cv, w.alpha, w.beta)
    out = Cd.cpu().numpy()
    del Ad, Bd, Cd
    return out


def check_pads(out, C_in, n, what):
    assert np.array_equal(out[:, n:], C_in[:, n:]), f"{what}: C padding written"
    assert np.all(np.isfinite(out[:, :n])), f"{what}: non-finite output (NaN pad read?)"


def full_check(orc, kind, w, integer):
    A, B, C = synth.operands(w, integer_twin=integer)
    say(kind, w.name, "int" if integer else "float")
    out = gpu_gemm(kind, w, A, B, C)
    check_pads(out, C, w.n, kind)
    ref = orc.sgemm(w.m, w.n, w.k, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, want_g=True)
    want = ref["C"].reshape(w.m, w.ldc)[:, :w.n]
    got = out[:, :w.n]
    if integer:
        assert_exact(got, want, f"{kind} {w.name} int")
    else:
        assert_close(got, want, ref["G"], w.alpha, w.beta, C[:, :w.n], f"{kind} {w.name}")


# The oracle's product for one (workload, twin), kept for the tests that follow
# (the paths of one workload run back to back); one entry at a time bounds the
# host memory (an 8192^2 result with its G is 0.75 GiB).
_REF = {}


def reference(orc, w, integer):
    """(A, B, C, oracle C over the logical m x n, G or None) of workload `w`."""
    key = (w, integer)
    if key not in _REF:
        _REF.clear()
        A, B, C = synth.operands(w, integer_twin=integer)
        say("oracle", w.name, "int" if integer else "float")
        ref = orc.sgemm(w.m, w.n, w.k, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc,
                        want_g=not integer)
        want = np.ascontiguousarray(ref["C"].reshape(w.m, w.ldc)[:, :w.n])
        _REF[key] = (A, B, C, want, ref["G"])
    return _REF[key]


def whole_check(orc, kind, w, integer):
    """Every output element of `kind` on workload `w` against the oracle."""
    A, B, C, want, G = reference(orc, w, integer)
    say(kind, w.name, "int" if integer else "float", "all elements")
    out = gpu_gemm(kind, w, A, B, C)
    check_pads(out, C, w.n, kind)
    got = out[:, :w.n]
    if integer:
        assert_exact(got, want, f"{kind} {w.name} int")
    else:
        assert_close_blocked(got, want, G, w.alpha, w.beta, C[:, :w.n], f"{kind} {w.name}")
    return out


# ---------------------------------------------------------------------------
# Small ragged shapes on every path and every tile configuration
# ---------------------------------------------------------------------------
KINDS = (["mfma", "valu", "valu_cfg0", "valu_cfg1", "splitk", "splitk3", "splitk1",
          "splitk_atomic", "splitk_atomic3"]
         + [f"mfma_cfg{i}" for i in range(N_MFMA_CFG)]
         + [f"splitk_cfg{i}" for i in range(N_MFMA_CFG)])
SHAPES = [(1, 1, 1), (7, 9, 5), (33, 65, 17), (130, 257, 300), (255, 129, 64), (64, 128, 2049)]


@pytest.mark.parametrize("ld_pad", [0, 3], ids=["ld=w", "ld=w+3"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("kind", KINDS)
def test_small_shapes(orc, kind, shape, ld_pad):
    m, n, k = shape
    base = synth.Workload(0, "small", m, n, k, k + ld_pad, n + ld_pad, n + ld_pad + 1,
                          "uniform", None, 1.0, 0.0)
    full_check(orc, kind, base, integer=False)
    wi = base.scaled(dist_c="int3", alpha=1.5, beta=0.5)
    full_check(orc, kind, wi, integer=True)


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["mfma", "valu", "splitk"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_256(orc, kind, integer):
    whole_check(orc, kind, synth.workload(0), integer)


@pytest.mark.parametrize("kind", ["mfma", "valu", "splitk"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_2048(orc, kind, integer):
    whole_check(orc, kind, synth.workload(1), integer)


@pytest.mark.parametrize("kind", ["mfma", "valu"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_8192_alpha_beta(orc, kind, integer):
    whole_check(orc, kind, synth.workload(2), integer)


@pytest.mark.parametrize("kind", ["mfma", "valu", "splitk"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_tails(orc, kind, integer):
    whole_check(orc, kind, synth.workload(3), integer)


@pytest.mark.parametrize("kind", ["splitk", "mfma", "splitk_atomic"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_workload_splitk(orc, kind, integer):
    whole_check(orc, kind, synth.workload(4), integer)


# ---------------------------------------------------------------------------
# Special cases of the interface
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["mfma", "valu", "splitk", "splitk_atomic"])
def test_beta_zero_ignores_nan_c(kind):
    say("beta0 nan C", kind)
    m, n, k = 70, 90, 33
    A = torch.ones((m, k), device="cuda")
    B = torch.ones((k, n), device="cuda")
    C = torch.full((m, n), float("nan"), device="cuda")
    run_kernel(kind, A, B, C, 2.0, 0.0)
    assert torch.equal(C, torch.full((m, n), 2.0 * k, device="cuda"))


@pytest.mark.parametrize("kind", ["mfma", "valu", "splitk", "splitk_atomic"])
def test_alpha_zero_and_k_zero(kind):
    say("alpha0/k0", kind)
    m, n = 45, 77
    g = torch.Generator(device="cpu").manual_seed(1)
    Cin = torch.randn((m, n), generator=g)
    A = torch.full((m, 8), float("nan"), device="cuda")
    B = torch.full((8, n), float("inf"), device="cuda")
    C = Cin.to("cuda")
    run_kernel(kind, A, B, C, 0.0, 0.75)
    want = (Cin.double() * 0.75).float()
    assert torch.equal(C.cpu(), want)
    C = Cin.to("cuda")
    run_kernel(kind, A[:, :0], B[:0, :], C, 1.0, -1.25)
    assert torch.equal(C.cpu(), (Cin.double() * -1.25).float())
    C = Cin.to("cuda")
    run_kernel(kind, A[:, :0], B[:0, :], C, 1.0, 0.0)
    assert torch.equal(C.cpu(), torch.zeros((m, n)))


@pytest.mark.parametrize("kind", ["mfma", "valu", "splitk", "splitk_atomic"])
def test_misaligned_operands(orc, kind):
    """Pointers one float off 16-byte alignment take the element-load path."""
    say("misaligned", kind)
    m, n, k = 97, 131, 203
    rng = np.random.default_rng(5)
    Ah = rng.integers(-3, 4, (m, k + 1)).astype(np.float32)
    Bh = rng.integers(-3, 4, (k, n + 1)).astype(np.float32)
    Ad = torch.from_numpy(Ah).cuda()
    Bd = torch.from_numpy(Bh).cuda()
    Cbig = torch.zeros((m * n + 1,), device="cuda")
    C = Cbig[1:].view(m, n)
    run_kernel(kind, Ad[:, 1:], Bd[:, 1:], C, 1.0, 0.0)
    want = (Ah[:, 1:].astype(np.int64) @ Bh[:, 1:].astype(np.int64)).astype(np.float32)
    assert_exact(C.cpu().numpy(), want, "misaligned")


@pytest.mark.parametrize("kind", ["mfma", "splitk"])
def test_deterministic(kind):
    say("determinism", kind)
    w = synth.workload(1)
    A, B, _ = synth.operands(w)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C1 = torch.empty((w.m, w.n), device="cuda")
    C2 = torch.empty((w.m, w.n), device="cuda")
    run_kernel(kind, Ad, Bd, C1, 1.0, 0.0)
    run_kernel(kind, Ad, Bd, C2, 1.0, 0.0)
    assert torch.equal(C1, C2)


def test_splitk_matches_unsplit(orc):
    say("splitk vs unsplit")
    w = synth.workload(3)
    A, B, C, _, G = reference(orc, w, False)
    out_s = gpu_gemm("splitk", w, A, B, C)
    out_u = gpu_gemm("mfma", w, A, B, C)
    # within tolerance of each other (twice the bar), every element
    assert_close_blocked(out_s[:, :w.n], out_u[:, :w.n], 2 * G, 1.0, 0.0, 0.0,
                         "split vs unsplit")


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 5, 7, 64])
def test_splitk_combine_partial_waves(splits):
    """Output counts that leave the last wave of the combine partly empty
    (m*n not a multiple of 64, nor of 4), split counts that are not multiples
    of the four lane groups: exact on integer operands."""
    say("combine", splits)
    rng = np.random.default_rng(splits)
    for (m, n, k) in [(7, 9, 640), (1, 3, 512), (13, 5, 1000)]:
        Ah = rng.integers(-3, 4, (m, k)).astype(np.float32)
        Bh = rng.integers(-3, 4, (k, n)).astype(np.float32)
        C = torch.zeros((m, n), device="cuda")
        s = min(splits, k)
        hta.sgemm_splitk(torch.from_numpy(Ah).cuda(), torch.from_numpy(Bh).cuda(), C,
                         1.0, 0.0, splits=s)
        torch.cuda.synchronize()
        want = (Ah.astype(np.int64) @ Bh.astype(np.int64)).astype(np.float32)
        assert_exact(C.cpu().numpy(), want, f"combine {m}x{n}x{k} s={s}")


def test_non_default_stream():
    say("stream")
    s = torch.cuda.Stream()
    m, n, k = 300, 200, 100
    A = torch.ones((m, k), device="cuda")
    B = torch.ones((k, n), device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = torch.empty((m, n), device="cuda")
        hta.sgemm(A, B, C, 1.0, 0.0)
        D = torch.empty((m, n), device="cuda")
        hta.sgemm_splitk(A, B, D, 1.0, 0.0, splits=4)
    s.synchronize()
    assert torch.equal(C, torch.full((m, n), float(k), device="cuda"))
    assert torch.equal(D, torch.full((m, n), float(k), device="cuda"))


def test_side_stream_allocations_not_reused_early():
    """stream= a side stream that is not torch's current one, with C and the
    workspace left to the helpers: they are allocated for the side stream, so
    the current stream's allocations and writes made while the kernels still
    run cannot land in them.  Integer-valued operands: exact results."""
    say("side stream, helper-allocated C and workspaces")
    rng = np.random.default_rng(21)
    m, n, k = 512, 512, 65536
    Ah, Bh = rng.integers(-3, 4, (m, k)).astype(np.float32), rng.integers(-3, 4, (k, n)).astype(np.float32)
    # Exact in float64 (integer products and partial sums below 9k < 2^53),
    # and a BLAS product: numpy's int64 product takes minutes at this size.
    want = (Ah.astype(np.float64) @ Bh.astype(np.float64)).astype(np.float32)
    xh = rng.integers(-3, 4, 1 << 22).astype(np.float32)
    A, B, x = torch.from_numpy(Ah).cuda(), torch.from_numpy(Bh).cuda(), torch.from_numpy(xh).cuda()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        # the side stream waits for nothing, so its kernels run while the
        # current stream allocates and overwrites memory below
        outs.append(("splitk", hta.sgemm_splitk(A, B, splits=16, stream=side)))
        outs.append(("streamk", hta.sgemm_streamk(A[:, :4096], B[:4096], stream=side)))
        outs.append(("sgemm", hta.sgemm(A[:, :2048], B[:2048], stream=side)))
        outs.append(("sum", hta.reduce_sum(x, stream=side)))
        junk = [torch.full((1 << 20,) if i % 2 else (m * n * 17,), float("nan"), device="cuda")
                for i in range(8)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    want_k = {
        "splitk": want,
        "streamk": (Ah[:, :4096].astype(np.float64) @ Bh[:4096].astype(np.float64)).astype(np.float32),
        "sgemm": (Ah[:, :2048].astype(np.float64) @ Bh[:2048].astype(np.float64)).astype(np.float32),
    }
    for name, got in outs:
        if name == "sum":
            assert float(got.item()) == float(xh.astype(np.int64).sum()), "side-stream reduce_sum"
        else:
            assert_exact(got.cpu().numpy(), want_k[name], f"side-stream {name}")


def test_splitk_atomic_beta_one_and_tolerance(orc):
    """beta == 1 skips the scaling pass (C accumulates in place); results of
    the atomic variant stay within the bar of the oracle."""
    say("splitk atomic beta=1")
    w = synth.workload(3).scaled(dist_c="uniform", alpha=-0.5, beta=1.0)
    whole_check(orc, "splitk_atomic", w, integer=False)
    whole_check(orc, "splitk_atomic", w, integer=True)


# ---------------------------------------------------------------------------
# Every ending of the k loop on every tile configuration
# ---------------------------------------------------------------------------
def k_loop_values(bk):
    """k values with 1..9 k steps of the tile, whole or with a partial last
    step: the steady loop stops one to five steps before the end, and the
    steps after it run as one of several fixed sequences chosen by how many
    steps remain and how many of them are whole."""
    return sorted({j * bk + r for j in range(9) for r in (1, bk - 1, bk) if j * bk + r > 0})


@pytest.mark.parametrize("aligned", [True, False], ids=["ld16B", "ld_odd"])
@pytest.mark.parametrize("config", range(N_MFMA_CFG))
def test_k_loop_endings(orc, config, aligned):
    bk = hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, config, 64, 64, 64, 0)["tile_k"]
    m, n = 70, 66
    for k in k_loop_values(bk):
        if aligned:
            lda, ldb = (k + 3) // 4 * 4 + 4, n + 2
        else:
            lda, ldb = (k + 1 if (k + 1) % 4 else k + 2), n + 1
        w = synth.Workload(9, "kloop", m, n, k, lda, ldb, n + 3, "uniform", "int3", 1.5, -0.5)
        full_check(orc, f"mfma_cfg{config}", w, integer=True)


def test_helper_argument_errors():
    """The torch helpers refuse what the C ABI cannot take, before any
    launch, and leave C untouched: wrong dtype, not 2-D, neither unit stride,
    inner sizes that differ, a C of the wrong shape, beta != 0 without C, and
    (VALU and atomic paths) a transposed view."""
    say("helper argument errors")
    A = torch.ones((8, 6), device="cuda")
    B = torch.ones((6, 4), device="cuda")
    C = torch.full((8, 4), 7.0, device="cuda")
    for fn in (hta.sgemm, hta.sgemm_valu, hta.sgemm_splitk, hta.sgemm_streamk,
               hta.sgemm_splitk_atomic):
        with pytest.raises(TypeError, match="float32"):
            fn(A.double(), B, C)
        with pytest.raises(ValueError, match="2-D"):
            fn(A.reshape(2, 4, 6), B, C)
        with pytest.raises(ValueError):
            fn(torch.ones((8, 12), device="cuda")[:, ::2], B, C)   # no unit stride
        with pytest.raises(ValueError, match="inner sizes"):
            fn(A, torch.ones((5, 4), device="cuda"), C)
        with pytest.raises(ValueError, match="expected"):
            fn(A, B, torch.empty((8, 5), device="cuda"))
        with pytest.raises(ValueError, match="needs C"):
            fn(A, B, None, 1.0, 0.5)
    for fn in (hta.sgemm_valu, hta.sgemm_splitk_atomic):
        with pytest.raises(ValueError, match="row-major"):
            fn(torch.ones((6, 8), device="cuda").t(), B, C)
    torch.cuda.synchronize()
    assert torch.equal(C, torch.full((8, 4), 7.0, device="cuda")), "C written by a refused call"
    # the transposed view is taken by the other entries
    hta.sgemm(torch.ones((6, 8), device="cuda").t(), B, C)
    torch.cuda.synchronize()
    assert torch.equal(C, torch.full((8, 4), 6.0, device="cuda"))

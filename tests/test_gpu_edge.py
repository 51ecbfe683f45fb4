"""Edge cases at extreme sizes, and use under HIP graph capture.

* Leading dimensions so large that a tile step's byte offsets leave the
  31-bit range of a buffer load: the vector kernels then stage every step
  through masked VGPR loads.  Checked bit-exact on integer operands, with
  NaN in the (huge) pads.
* Very tall or very wide products and a k of 2^24 (the largest k for which
  an all-ones product is exact in float).
* Calls captured into a HIP graph (through torch.cuda.graph) and replayed
  several times, with eager work in between: every replay equals the eager
  result.
"""
import numpy as np
import pytest

from parity import assert_exact

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import hpc_tiling_amd as hta
else:
    hta = None


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def ints(rng, shape):
    return rng.integers(-3, 4, shape).astype(np.float32)


def padded_device(values, ld):
    """A rows x ld device tensor, NaN outside the logical block."""
    rows, cols = values.shape
    t = torch.full((rows, ld), float("nan"), device="cuda")
    t[:, :cols] = torch.from_numpy(values).cuda()
    return t


def exact_product(Ah, Bh):
    return (Ah.astype(np.int64) @ Bh.astype(np.int64)).astype(np.float32)


@pytest.mark.parametrize("which", ["A", "B", "A^T"])
def test_leading_dimension_beyond_direct_load_range(which):
    """lda >= 2^31 / (4 * 64) floats for A (rows of a 64-row tile step span
    more than 2^31 bytes), ldb >= 2^31 / (4 * 32) for B (32 k rows)."""
    rng = np.random.default_rng(3)
    m, n, k = 5, 70, 64
    Ah, Bh = ints(rng, (m, k)), ints(rng, (k, n))
    want = exact_product(Ah, Bh)
    say("huge ld", which)
    C = torch.zeros((m, n), device="cuda")
    if which == "A":
        A = padded_device(Ah, 9_000_000)[:, :k]
        B = torch.from_numpy(Bh).cuda()
    elif which == "B":
        A = torch.from_numpy(Ah).cuda()
        B = padded_device(Bh, 17_000_000)[:, :n]
    else:  # A stored transposed (k x m) with a huge row stride
        A = padded_device(np.ascontiguousarray(Ah.T), 17_000_000)[:, :m].t()
        B = torch.from_numpy(Bh).cuda()
    for config in (None, 6, 9):
        C.zero_()
        hta.sgemm(A, B, C, config=config)
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), want, f"huge ld {which} config {config}")
    del A, B
    torch.cuda.empty_cache()


# k values whose step counts (9, 10, 18, 19, 28 and 37 steps of 16 or 32)
# once made the last steps of a tile alias another compile-time tail when
# direct loads are off, so that steps were skipped.
HUGE_LDA_K = (140, 155, 270, 285, 300, 445, 570, 590, 600, 890, 1180)


@pytest.mark.parametrize("config", [0, 6, 9, 12, 13, 14])
def test_long_k_without_direct_loads(config):
    """lda = 9e6 floats puts a tile step of A past the 2^31-byte range of a
    direct load for every tile height used (64 and 128 rows), so every step
    loads through VGPRs, decided at run time, and the last steps take the
    run-time tail.  Three-buffer (0, 6, 12) and four-buffer (9, 13, 14)
    rings, over k values with many step counts, bit-exact on integers."""
    rng = np.random.default_rng(4)
    m, n, kmax = 5, 70, max(HUGE_LDA_K)
    Ah, Bh = ints(rng, (m, kmax)), ints(rng, (kmax, n))
    A_all = padded_device(Ah, 9_000_000)
    B_all = torch.from_numpy(Bh).cuda()
    for k in HUGE_LDA_K:
        say("huge lda, config", config, "k", k)
        C = hta.sgemm(A_all[:, :k], B_all[:k], config=config)
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), exact_product(Ah[:, :k], Bh[:k]),
                     f"huge lda, config {config}, k {k}")
    del A_all, B_all
    torch.cuda.empty_cache()


@pytest.mark.parametrize("config", [6, 9, 14])
def test_streamk_long_k_without_direct_loads(config):
    """The same operands through a forced stream-K schedule of 3 workgroups:
    every segment's step count goes through the same tail dispatch."""
    rng = np.random.default_rng(5)
    m, n, kmax = 5, 70, max(HUGE_LDA_K)
    Ah, Bh = ints(rng, (m, kmax)), ints(rng, (kmax, n))
    A_all = padded_device(Ah, 9_000_000)
    B_all = torch.from_numpy(Bh).cuda()
    for k in HUGE_LDA_K:
        say("huge lda, stream-K, config", config, "k", k)
        C = hta.sgemm_streamk(A_all[:, :k], B_all[:k], grid=3, config=config)
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), exact_product(Ah[:, :k], Bh[:k]),
                     f"huge lda, stream-K, config {config}, k {k}")
    del A_all, B_all
    torch.cuda.empty_cache()


@pytest.mark.parametrize("config", [6, 9, 13])
def test_splitk_long_k_without_direct_loads(config):
    """The same operands through split-K partial slices (2 to 7 slices of
    k = 1180): each slice's step count goes through the same tail dispatch."""
    rng = np.random.default_rng(6)
    m, n, k = 5, 70, 1180
    Ah, Bh = ints(rng, (m, k)), ints(rng, (k, n))
    A = padded_device(Ah, 9_000_000)[:, :k]
    B = torch.from_numpy(Bh).cuda()
    want = exact_product(Ah, Bh)
    for splits in (2, 3, 5, 7):
        say("huge lda, split-K, config", config, "splits", splits)
        C = hta.sgemm_splitk(A, B, splits=splits, config=config)
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), want, f"huge lda, split-K, config {config}, {splits} slices")
    del A, B
    torch.cuda.empty_cache()


def test_valu_long_k_huge_lda():
    """The register-tiled VALU kernel with lda = 9e6 floats (its offsets are
    64-bit) over the same k values."""
    rng = np.random.default_rng(7)
    m, n, kmax = 5, 70, max(HUGE_LDA_K)
    Ah, Bh = ints(rng, (m, kmax)), ints(rng, (kmax, n))
    A_all = padded_device(Ah, 9_000_000)
    B_all = torch.from_numpy(Bh).cuda()
    for k in HUGE_LDA_K:
        say("huge lda, VALU, k", k)
        C = hta.sgemm_valu(A_all[:, :k], B_all[:k])
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), exact_product(Ah[:, :k], Bh[:k]), f"huge lda, VALU, k {k}")
    del A_all, B_all
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", [(1_000_000, 8, 16), (8, 1_000_000, 16), (3, 3, 1_000_003)],
                         ids=["tall", "wide", "long-k"])
def test_extreme_aspect_ratios(shape):
    m, n, k = shape
    rng = np.random.default_rng(5)
    Ah, Bh = ints(rng, (m, k)), ints(rng, (k, n))
    say("aspect", shape)
    want = exact_product(Ah, Bh)
    A, B = torch.from_numpy(Ah).cuda(), torch.from_numpy(Bh).cuda()
    C = torch.empty((m, n), device="cuda")
    hta.sgemm(A, B, C)
    torch.cuda.synchronize()
    assert_exact(C.cpu().numpy(), want, f"mfma {shape}")
    D = torch.empty((m, n), device="cuda")
    hta.sgemm_splitk(A, B, D, splits=0)
    torch.cuda.synchronize()
    assert_exact(D.cpu().numpy(), want, f"splitk {shape}")


def test_k_two_to_the_24_all_ones():
    """2^24 is the largest count of ones a float sums exactly; both the
    single-pass and split-K paths must reach it."""
    k = 1 << 24
    say("k=2^24")
    A = torch.ones((2, k), device="cuda")
    B = torch.ones((k, 3), device="cuda")
    C = torch.empty((2, 3), device="cuda")
    hta.sgemm(A, B, C)
    D = torch.empty((2, 3), device="cuda")
    hta.sgemm_splitk(A, B, D, splits=0)
    torch.cuda.synchronize()
    assert torch.equal(C, torch.full((2, 3), float(k), device="cuda"))
    assert torch.equal(D, torch.full((2, 3), float(k), device="cuda"))


def test_graph_capture_replay():
    """mi_sgemm, mi_sgemm_splitk (with its workspace) and mi_reduce_sum
    captured into one graph; inputs changed eagerly between replays."""
    say("graph capture")
    rng = np.random.default_rng(7)
    m, n, k = 300, 200, 1000
    A = torch.from_numpy(ints(rng, (m, k))).cuda()
    B = torch.from_numpy(ints(rng, (k, n))).cuda()
    C = torch.empty((m, n), device="cuda")
    D = torch.empty((m, n), device="cuda")
    x = torch.from_numpy(ints(rng, (1 << 20,)).reshape(-1)).cuda()
    s = torch.empty(1, device="cuda")
    ws = hta.splitk_workspace(m, n, k, 8)
    rws = torch.empty(max(hta.mi_reduce_sum_workspace_bytes(x.numel()), 4), dtype=torch.uint8,
                      device="cuda")
    # first calls eagerly (the library checks the device once, outside capture)
    hta.sgemm(A, B, C)
    hta.sgemm_splitk(A, B, D, splits=8, workspace=ws)
    hta.reduce_sum(x, out=s, workspace=rws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            hta.sgemm(A, B, C, 1.0, 0.0)
            hta.sgemm_splitk(A, B, D, 1.0, 0.0, splits=8, workspace=ws)
            hta.reduce_sum(x, out=s, workspace=rws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        # eager work between replays: new inputs, and the outputs scribbled over
        A.copy_(torch.from_numpy(ints(rng, (m, k))).cuda())
        x.copy_(torch.from_numpy(ints(rng, (1 << 20,)).reshape(-1)).cuda())
        C.fill_(float("nan"))
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = exact_product(A.cpu().numpy(), B.cpu().numpy())
        assert_exact(C.cpu().numpy(), want, f"graph replay {rep} mfma")
        assert_exact(D.cpu().numpy(), want, f"graph replay {rep} splitk")
        assert s.item() == float(x.cpu().double().sum()), f"graph replay {rep} reduce"


def test_noalloc_entry_under_graph_capture():
    """The allocation-free split-K entry (its partial sums in the library's
    static scratch) captured into a graph -- the use it exists for -- and
    replayed with new inputs between replays: every replay equals the
    integer product, and equals the entry with a caller workspace."""
    say("graph capture noalloc")
    rng = np.random.default_rng(8)
    m, n, k = 260, 190, 3000
    A = torch.from_numpy(ints(rng, (m, k))).cuda()
    B = torch.from_numpy(ints(rng, (k, n))).cuda()
    C = torch.empty((m, n), device="cuda")
    args = lambda stream: (0, 0, m, n, k, 1.0, A.data_ptr(), k, B.data_ptr(), n, 0.0,
                           C.data_ptr(), n, 6, stream)
    # the first call on the device sets the scratch up, outside capture
    assert hta.mi_sgemm_splitk_noalloc(*args(torch.cuda.current_stream().cuda_stream)) == hta.SUCCESS
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            st = hta.mi_sgemm_splitk_noalloc(*args(side.cuda_stream))
    assert st == hta.SUCCESS
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        A.copy_(torch.from_numpy(ints(rng, (m, k))).cuda())
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert_exact(got, exact_product(A.cpu().numpy(), B.cpu().numpy()), f"noalloc replay {rep}")
        D = hta.sgemm_splitk(A, B, splits=6)
        torch.cuda.synchronize()
        assert np.array_equal(got, D.cpu().numpy()), f"noalloc replay {rep} vs workspace entry"


def test_concurrent_host_threads_and_streams():
    """Four host threads, each with its own stream and workspace, call the
    library at the same time (ctypes releases the GIL around each call); the
    library holds no per-call global state, so every result is exact."""
    import threading
    say("threads x streams")
    rng = np.random.default_rng(13)
    shapes = [(300, 200, 257), (129, 511, 64), (64, 64, 4096), (1000, 33, 100)]
    cases = []
    for (m, n, k) in shapes:
        Ah, Bh = ints(rng, (m, k)), ints(rng, (k, n))
        cases.append((torch.from_numpy(Ah).cuda(), torch.from_numpy(Bh).cuda(), exact_product(Ah, Bh)))
    torch.cuda.synchronize()
    errors = []

    def worker(idx):
        try:
            A, B, want = cases[idx]
            m, n, k = A.shape[0], B.shape[1], A.shape[1]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                ws = hta.splitk_workspace(m, n, k, 3)
                outs = []
                for rep in range(10):
                    C = torch.empty((m, n), device="cuda")
                    if rep % 2:
                        hta.sgemm_splitk(A, B, C, splits=3, workspace=ws)
                    else:
                        hta.sgemm(A, B, C)
                    outs.append(C)
            stream.synchronize()
            for rep, C in enumerate(outs):
                if not np.array_equal(C.cpu().numpy(), want):
                    errors.append(f"thread {idx} call {rep} differs")
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(f"thread {idx}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


def test_launch_beyond_32bit_work_items_refused():
    """A dispatch holds its grid size in work-items as 32 bits.  Atomic
    split-K at 16384^2 x 32768 with 1024 forced slices plans 2^24 workgroups
    of 256 lanes, i.e. 2^32 work-items: the call is refused with
    INVALID_VALUE before C is scaled, and C keeps its values.  (The operands
    are real buffers of the full size, so a launch could only compute.)"""
    m = n = 16384
    k, splits = 32768, 1024
    plan = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK_ATOMIC, -1, m, n, k, splits)
    assert plan["workgroups"] * plan["threads"] > 2**32 - 1
    say("refused launch", m, n, k, splits, plan["workgroups"], plan["threads"])
    A = torch.zeros((m, k), device="cuda")
    B = torch.zeros((k, n), device="cuda")
    C = torch.full((m, n), 7.0, device="cuda")
    st = hta.mi_sgemm_splitk_atomic(m, n, k, 1.0, A.data_ptr(), k, B.data_ptr(), n, 0.5,
                                    C.data_ptr(), n, splits)
    torch.cuda.synchronize()
    assert st == hta.ERROR_INVALID_VALUE
    assert bool((C == 7.0).all())
    del A, B, C
    torch.cuda.empty_cache()


def test_splitk_combine_past_its_block_cap():
    """The combine kernel caps its grid at 2^20 blocks of four waves and walks
    the rest of the 64-output chunks grid-stride: 16384 x 16400 has 1049600
    blocks' worth, so the last 1024 blocks' chunks (the last rows of C) are
    done on a second pass.  Integer operands: every element equals the
    single-pass result, and sampled rows (the last 16 among them) equal the
    exact integer product."""
    rng = np.random.default_rng(12)
    m, n, k = 16384, 16400, 64
    plan = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, m, n, k, 2)
    assert plan["splits"] == 2 and plan["stream_k_grid"] == 0
    say("combine past cap", m, n, k)
    Ah, Bh = ints(rng, (m, k)), ints(rng, (k, n))
    A, B = torch.from_numpy(Ah).cuda(), torch.from_numpy(Bh).cuda()
    C = torch.empty((m, n), device="cuda")
    hta.sgemm_splitk(A, B, C, splits=2)
    C1 = hta.sgemm(A, B)
    torch.cuda.synchronize()
    assert torch.equal(C, C1)
    rows = np.concatenate([np.arange(0, m, 997), np.arange(m - 16, m)])
    got = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert_exact(got, exact_product(Ah[rows], Bh), "combine past its block cap")
    del A, B, C, C1
    torch.cuda.empty_cache()


@pytest.mark.parametrize("config", [-1, 0, 6, 9, 13, 14])
def test_workgroup_order_is_bitwise_neutral(config):
    """The workgroup order only decides which workgroup computes which tile:
    every (XCD remap, group height) gives the bits of the default order,
    including group heights that do not divide the tile rows."""
    say("order", config)
    m, n, k = 1000, 777, 333
    rng = np.random.default_rng(21)
    A = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).cuda()
    B = torch.from_numpy(rng.standard_normal((k, n)).astype(np.float32)).cuda()
    C0 = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).cuda()
    cfg = None if config < 0 else config
    ref = hta.sgemm(A, B, C0.clone(), 1.25, -0.5, config=cfg)
    for order in [(1, 8), (0, 8), (1, 1), (0, 1), (0, 3), (1, 5), (1, 1000)]:
        got = hta.sgemm(A, B, C0.clone(), 1.25, -0.5, config=cfg, order=order)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"order {order} config {config}"


def test_clock_and_fma_probes():
    """The measurement helpers run and report plausible figures: a core clock
    between 100 and 3000 MHz on every XCD, and finite outputs of both FMA
    loops."""
    say("probes")
    probe = hta.ClockProbe()
    probe.launch()
    torch.cuda.synchronize()
    mhz = probe.mhz()
    assert len(mhz) == 8 and all(100 < x < 3000 for x in mhz), mhz
    out = torch.full((256 * 64,), float("nan"), device="cuda")
    for loop in (0, 1):
        assert hta.mi_fma_rate_probe(loop, out.data_ptr(), 64, 10) == hta.SUCCESS
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        out.fill_(float("nan"))

"""mi_sgemm_splitk_noalloc: the split-K entry point that allocates nothing,
its workspace a static 64 MiB device scratch buffer.

GPU: through the C ABI (raw device pointers, no allocation inside the call),
its results equal those of mi_sgemm_splitk_ex with a caller workspace --
bitwise where both run the same plan, within the tolerance of tests/parity.py
and bit-exact on integer operands otherwise -- on two calls in a row, the
second smaller (the scratch keeps the first call's contents).  Host: a forced
plan beyond the scratch is refused before anything is enqueued.
"""
import numpy as np
import pytest

import synth
from parity import assert_close, assert_exact

torch = pytest.importorskip("torch")
import hpc_tiling_amd as hta  # noqa: E402

P = 0x10000  # never-dereferenced address for the host-side checks
_SET_UP = [False]  # a call has run on the GPU in this process


def say(*a):
    print("[case]", *a, flush=True)


def test_forced_plan_beyond_scratch_refused():
    """8 slices of a 2048 x 2048 C need 128 MiB: refused on the host."""
    f = hta.mi_sgemm_splitk_noalloc
    need = hta.mi_sgemm_splitk_workspace_bytes(2048, 2048, 4096, 8)
    assert need > hta.NOALLOC_SCRATCH_BYTES
    st = f(0, 0, 2048, 2048, 4096, 1.0, P, 4096, P, 2048, 0.0, P, 2048, 8, None)
    assert st == hta.ERROR_SCRATCH_LIMIT
    assert "64 MiB" in hta.mi_status_string(st)
    # argument errors come first, as in mi_sgemm_splitk_ex
    assert f(0, 0, -1, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4, 0, None) == hta.ERROR_INVALID_VALUE
    assert f(0, 0, 4, 4, 4, 1.0, P, 3, P, 4, 0.0, P, 4, 0, None) == hta.ERROR_INVALID_LD
    assert f(0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, None, 4, 0, None) == hta.ERROR_NULL_POINTER
    assert f(0, 0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 0, None) == hta.SUCCESS


def _ptrs(w, integer, ta=0, tb=0):
    A, lda, B, ldb, C = synth.operands_ex(w, ta, tb, integer_twin=integer)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C1 = torch.from_numpy(C).cuda()
    C2 = C1.clone()
    return (A, lda, B, ldb, C), (Ad, Bd, C1, C2)


def _compare(w, integer, ta=0, tb=0, splits=0):
    (A, lda, B, ldb, C), (Ad, Bd, C1, C2) = _ptrs(w, integer, ta, tb)
    nbytes = hta.mi_sgemm_splitk_workspace_bytes(w.m, w.n, w.k, splits)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    st = hta.mi_sgemm_splitk_ex(ta, tb, w.m, w.n, w.k, w.alpha, Ad.data_ptr(), lda, Bd.data_ptr(),
                                ldb, w.beta, C1.data_ptr(), w.ldc, splits, ws.data_ptr(), nbytes, s)
    assert st == hta.SUCCESS, hta.mi_status_string(st)
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    st = hta.mi_sgemm_splitk_noalloc(ta, tb, w.m, w.n, w.k, w.alpha, Ad.data_ptr(), lda,
                                     Bd.data_ptr(), ldb, w.beta, C2.data_ptr(), w.ldc, splits, s)
    assert st == hta.SUCCESS, hta.mi_status_string(st)
    torch.cuda.synchronize()
    # Nothing is allocated on the device by a call once the scratch is set up
    # (the first call on a device looks up its address; the runtime may take
    # memory for its own bookkeeping then).
    if _SET_UP[0]:
        assert torch.cuda.mem_get_info()[0] == free_before, "device memory allocated"
    _SET_UP[0] = True
    got, want = C2.cpu().numpy(), C1.cpu().numpy()
    assert np.array_equal(got[:, w.n:], C[:, w.n:]), "C padding written"
    return got[:, :w.n], want[:, :w.n], C, nbytes


CASES = [
    # (name, workload, transposes, split request), each call smaller than the
    # one before (the scratch keeps the previous call's partial sums).  The
    # first one's automatic plan needs 79 MiB of workspace: the allocation-free
    # entry runs a plan that fits instead (another summation order).
    ("896x896x65536, auto plan beyond the scratch",
     synth.Workload(30, "n0", 896, 896, 65536, 65536, 896, 896, "uniform", None, 1.0, 0.0),
     (0, 0), 0),
    ("stream-K 1536x1536x4096", synth.workload(5), (0, 0), 0),
    ("ragged 300x200x5000 TN, 3 slices",
     synth.Workload(31, "na", 300, 200, 5000, 5003, 203, 205, "uniform", "normal", 1.25, -0.5),
     (1, 0), 3),
    ("ragged 70x33x999 NT, auto",
     synth.Workload(32, "nb", 70, 33, 999, 1001, 35, 34, "uniform", "normal", 0.5, 2.0),
     (0, 1), 0),
]


def _check_cases(orc, cases, integer):
    for name, w, (ta, tb), splits in cases:
        say("noalloc", name, "int" if integer else "float")
        got, want, C, nbytes = _compare(w, integer, ta, tb, splits)
        if nbytes <= hta.NOALLOC_SCRATCH_BYTES or integer:
            # the same plan (same bits), or integer sums (exact in any order)
            assert_exact(got, want, f"noalloc {name}")
        else:
            A, lda, B, ldb, _ = synth.operands_ex(w, ta, tb)
            ref = orc.sgemm(w.m, w.n, w.k, w.alpha, A, lda, B, ldb, w.beta, C, w.ldc,
                            want_g=True, trans_a=bool(ta), trans_b=bool(tb))
            exp = ref["C"].reshape(w.m, w.ldc)[:, :w.n]
            for out, who in ((got, "noalloc"), (want, "workspace entry")):
                assert_close(out, exp, ref["G"], w.alpha, w.beta, C[:, :w.n], f"{who} {name}")


@pytest.mark.gpu
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
def test_noalloc_matches_workspace_entry(orc, integer):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _check_cases(orc, CASES, integer)


@pytest.mark.gpu
def test_noalloc_splitk_workload_then_smaller(orc):
    """The 512 x 512 x 262144 split-K workload (16 slices, 16 MiB of
    scratch), then a smaller call on the same scratch."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _check_cases(orc, [("splitk 512x512x262144", synth.workload(4), (0, 0), 0), CASES[2]], False)

"""Host-side checks of the C-ABI library: it loads, exports every function the
header declares, plans launches as the pages' worked example says, and rejects
bad arguments before touching any GPU.  No compute call runs here."""
import ctypes
import re
from pathlib import Path

import pytest

import hpc_tiling_amd as hta

ROOT = Path(__file__).resolve().parents[1]
GOLDEN = Path(__file__).resolve().parent / "golden"


def _declared_functions():
    names = set()
    for h in (ROOT / "include").glob("*.h"):
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(mi_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def _golden(name):
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        out[parts[0]] = parts[1:] if len(parts) > 2 else parts[1]
    return out


def test_header_declares_expected_functions():
    assert _declared_functions() == set(hta.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(str(hta.LIB_PATH))
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings():
    for st in range(7):
        assert hta.mi_status_string(st) != "unknown status"
    assert hta.mi_status_string(99) == "unknown status"


def test_valu_plan_is_the_worked_example():
    g = {k: int(v) for k, v in _golden("worked_example_2048.txt").items()}
    p = hta.mi_sgemm_get_plan(hta.KERNEL_VALU, 0, g["m"], g["n"], g["k"])
    for key in ("tile_m", "tile_n", "tile_k", "micro_m", "micro_n", "workgroups", "threads",
                "outputs_per_thread", "big_iterations", "small_iterations",
                "fma_per_small_iteration", "a_elements_per_big_iteration",
                "b_elements_per_big_iteration"):
        assert p[key] == g[key], key
    assert p["tile_m"] * p["tile_n"] == g["c_elements_per_block"]


def test_valu_automatic_k_groups():
    """The automatic VALU plan splits each tile over two k groups while no CU
    gets a second workgroup (at most 256 tiles), and keeps the worked
    example's 256 threads otherwise."""
    assert hta.mi_sgemm_config_count(hta.KERNEL_VALU) == 2
    for (m, n, k, cfg, threads) in [(2048, 2048, 2048, 1, 512), (256, 256, 256, 1, 512),
                                    (2048, 2049, 64, 0, 256), (4096, 4096, 4096, 0, 256),
                                    (128 * 16, 128 * 16, 7, 1, 512), (128 * 16 + 1, 128 * 16, 7, 0, 256)]:
        p = hta.mi_sgemm_get_plan(hta.KERNEL_VALU, -1, m, n, k)
        assert (p["config"], p["threads"]) == (cfg, threads), (m, n, k)
        assert p["workgroups"] == -(-m // 128) * -(-n // 128)
    assert hta.mi_sgemm_get_plan(hta.KERNEL_VALU, 1, 4096, 4096, 8)["threads"] == 512


def test_mfma_plan_geometry():
    for cfg in range(hta.mi_sgemm_config_count(hta.KERNEL_MFMA)):
        p = hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, cfg, 3001, 4997, 1023)
        assert p["tiles_m"] == -(-3001 // p["tile_m"])
        assert p["tiles_n"] == -(-4997 // p["tile_n"])
        assert p["workgroups"] == p["tiles_m"] * p["tiles_n"]
        assert p["big_iterations"] == -(-1023 // p["tile_k"])
        assert p["micro_m"] % 32 == 0 and p["micro_n"] % 32 == 0
        assert p["threads"] % 64 == 0
        waves = p["threads"] // 64
        assert p["outputs_per_thread"] * 64 * waves == p["tile_m"] * p["tile_n"]


def test_splitk_plan_and_workspace():
    p = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, 512, 512, 262144, 0)
    assert p["splits"] * p["k_per_split"] >= 262144
    assert (p["splits"] - 1) * p["k_per_split"] < 262144
    assert p["k_per_split"] % p["tile_k"] == 0
    ws = hta.mi_sgemm_splitk_workspace_bytes(512, 512, 262144, 0)
    assert ws == p["workspace_bytes"] >= p["splits"] * 512 * 512 * 4
    # explicit split counts: never more slices than asked, each slice whole k steps
    for req in (1, 2, 3, 7, 64, 1000):
        q = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, 100, 70, 5000, req)
        assert 1 <= q["splits"] <= req
        assert q["splits"] * q["k_per_split"] >= 5000 > (q["splits"] - 1) * q["k_per_split"]
    assert hta.mi_sgemm_splitk_workspace_bytes(4, 4, 8, 9) == 0   # splits > k
    assert hta.mi_sgemm_splitk_workspace_bytes(0, 4, 8, 0) == 0
    assert hta.mi_sgemm_splitk_workspace_bytes(4, 4, 0, 0) == 0


def test_bad_plan_requests():
    with pytest.raises(hta.MiSgemmError):
        hta.mi_sgemm_get_plan(7, -1, 1, 1, 1)
    with pytest.raises(hta.MiSgemmError):
        hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, 99, 1, 1, 1)
    with pytest.raises(hta.MiSgemmError):
        hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, -1, -1, 1, 1)


# Fake, never-dereferenced device addresses: every call below must return an
# error (or a no-op) before anything is enqueued.
P = 0x10000


@pytest.mark.parametrize("fn", [hta.mi_sgemm, hta.mi_sgemm_valu])
def test_argument_errors(fn):
    E = hta
    assert fn(-1, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert fn(4, -1, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert fn(4, 4, -1, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert fn(4, 4, 8, 1.0, P, 7, P, 4, 0.0, P, 4) == E.ERROR_INVALID_LD
    assert fn(4, 6, 8, 1.0, P, 8, P, 5, 0.0, P, 6) == E.ERROR_INVALID_LD
    assert fn(4, 6, 8, 1.0, P, 8, P, 6, 0.0, P, 5) == E.ERROR_INVALID_LD
    assert fn(4, 4, 4, 1.0, P, 4, P, 4, 0.0, None, 4) == E.ERROR_NULL_POINTER
    assert fn(4, 4, 4, 1.0, None, 4, P, 4, 0.0, P, 4) == E.ERROR_NULL_POINTER
    assert fn(4, 4, 4, 1.0, P, 4, None, 4, 0.0, P, 4) == E.ERROR_NULL_POINTER
    # nothing to do: success without touching any pointer or device
    assert fn(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4) == E.SUCCESS
    assert fn(4, 0, 4, 1.0, None, 4, None, 1, 0.0, None, 1) == E.SUCCESS


def test_splitk_argument_errors():
    E, f = hta, hta.mi_sgemm_splitk
    ws = hta.mi_sgemm_splitk_workspace_bytes(64, 64, 1024, 0)
    assert f(64, 64, 1024, 1.0, P, 1024, P, 64, 0.0, P, 64, -1, P, ws) == E.ERROR_INVALID_VALUE
    assert f(64, 64, 1024, 1.0, P, 1024, P, 64, 0.0, P, 64, 1025, P, ws) == E.ERROR_INVALID_VALUE
    assert f(64, 64, 1024, 1.0, P, 1000, P, 64, 0.0, P, 64, 0, P, ws) == E.ERROR_INVALID_LD
    assert f(64, 64, 1024, 1.0, P, 1024, P, 64, 0.0, P, 64, 0, P, ws - 1) == E.ERROR_WORKSPACE
    assert f(64, 64, 1024, 1.0, P, 1024, P, 64, 0.0, P, 64, 0, None, ws) == E.ERROR_WORKSPACE
    assert f(64, 64, 1024, 1.0, None, 1024, P, 64, 0.0, P, 64, 0, P, ws) == E.ERROR_NULL_POINTER
    assert f(0, 64, 1024, 1.0, None, 1024, None, 64, 0.0, None, 64, 0, None, 0) == E.SUCCESS


def test_probe_argument_errors():
    E = hta
    f = hta.mi_fma_rate_probe
    assert f(2, P, 1, 1) == E.ERROR_INVALID_VALUE
    assert f(0, P, 0, 1) == E.ERROR_INVALID_VALUE
    assert f(1, P, 1, 0) == E.ERROR_INVALID_VALUE
    assert f(0, None, 1, 1) == E.ERROR_NULL_POINTER
    assert f(0, P, 1, 1) == E.ERROR_DEVICE
    ref = ctypes.c_int(0)
    g = hta.mi_clock_probe
    assert g(P, 0, 20, ref) == E.ERROR_INVALID_VALUE
    assert g(P, 1025, 20, ref) == E.ERROR_INVALID_VALUE
    assert g(P, 8, 0, ref) == E.ERROR_INVALID_VALUE
    assert g(None, 8, 20, ref) == E.ERROR_NULL_POINTER
    assert g(P, 8, 20, ref) == E.ERROR_DEVICE


def test_order_argument_errors():
    E, f = hta, hta.mi_sgemm_with_order
    assert f(-1, 2, 8, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert f(-1, 1, 0, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert f(99, 1, 8, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert f(-1, 0, 1, 0, 0, 4, 4, 4, 1.0, P, 3, P, 4, 0.0, P, 4) == E.ERROR_INVALID_LD
    assert f(-1, 0, 1, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == E.ERROR_DEVICE


def test_splitk_combine_argument_errors():
    """The combine entry checks sizes, ld, pointers and the slice layout (a
    multiple of 4 floats, at least m*n rounded up to 4, 16-byte aligned
    partials) before anything else."""
    E, f = hta, hta.mi_sgemm_splitk_combine
    assert f(-1, 4, 2, P, 16, 1.0, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert f(4, -1, 2, P, 16, 1.0, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert f(4, 4, -1, P, 16, 1.0, 0.0, P, 4) == E.ERROR_INVALID_VALUE
    assert f(4, 4, 2, P, 16, 1.0, 0.0, P, 3) == E.ERROR_INVALID_LD
    assert f(4, 4, 2, P, 16, 1.0, 0.0, None, 4) == E.ERROR_NULL_POINTER
    assert f(4, 4, 2, None, 16, 1.0, 0.0, P, 4) == E.ERROR_NULL_POINTER
    assert f(4, 4, 2, P, 18, 1.0, 0.0, P, 4) == E.ERROR_INVALID_VALUE   # slice % 4
    assert f(5, 3, 2, P, 12, 1.0, 0.0, P, 3) == E.ERROR_INVALID_VALUE   # 15 > 12
    assert f(4, 4, 2, P + 4, 16, 1.0, 0.0, P, 4) == E.ERROR_INVALID_VALUE   # unaligned
    assert f(0, 4, 2, None, 0, 1.0, 0.0, None, 4) == E.SUCCESS
    # a valid call reaches the device check (none here)
    assert f(5, 3, 2, P, 16, 1.0, 0.0, P, 3) == E.ERROR_DEVICE


def test_splitk_atomic_argument_errors():
    E, f = hta, hta.mi_sgemm_splitk_atomic
    assert f(-1, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4, 0) == E.ERROR_INVALID_VALUE
    assert f(4, 4, 8, 1.0, P, 8, P, 4, 0.0, P, 4, 9) == E.ERROR_INVALID_VALUE   # splits > k
    assert f(4, 4, 8, 1.0, P, 8, P, 4, 0.0, P, 4, -1) == E.ERROR_INVALID_VALUE
    assert f(4, 4, 8, 1.0, P, 7, P, 4, 0.0, P, 4, 0) == E.ERROR_INVALID_LD
    assert f(4, 4, 8, 1.0, P, 8, P, 4, 0.0, None, 4, 0) == E.ERROR_NULL_POINTER
    assert f(0, 4, 8, 1.0, None, 8, None, 4, 0.0, None, 4, 0) == E.SUCCESS
    p = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK_ATOMIC, -1, 512, 512, 262144, 0)
    q = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, 512, 512, 262144, 0)
    assert p["workspace_bytes"] == 0 and p["splits"] == q["splits"] > 1


def test_with_config_rejects_unknown_ids():
    n = hta.mi_sgemm_config_count(hta.KERNEL_MFMA)
    assert n >= 1
    r = hta.mi_sgemm_with_config(hta.KERNEL_MFMA, n, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert r == hta.ERROR_INVALID_VALUE
    nv = hta.mi_sgemm_config_count(hta.KERNEL_VALU)
    r = hta.mi_sgemm_with_config(hta.KERNEL_VALU, nv, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert r == hta.ERROR_INVALID_VALUE
    r = hta.mi_sgemm_with_config(5, 0, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert r == hta.ERROR_INVALID_VALUE
    # the VALU kernel takes operands as given only
    r = hta.mi_sgemm_with_config(hta.KERNEL_VALU, 0, 1, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert r == hta.ERROR_INVALID_VALUE
    r = hta.mi_sgemm_splitk_with_config(n, 0, 0, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4, 0, P, 1 << 20)
    assert r == hta.ERROR_INVALID_VALUE


@pytest.mark.parametrize("entry", ["ex", "splitk_ex"])
def test_transpose_argument_errors(entry):
    """Leading dimensions are checked against the stored row width: k for A
    and n for B as given, m for A^T and k for B^T; flags must be 0 or 1."""
    E = hta
    ws = 1 << 20

    def f(ta, tb, m, n, k, lda, ldb, ldc, A=P, B=P, C=P):
        if entry == "ex":
            return hta.mi_sgemm_ex(ta, tb, m, n, k, 1.0, A, lda, B, ldb, 0.0, C, ldc)
        return hta.mi_sgemm_splitk_ex(ta, tb, m, n, k, 1.0, A, lda, B, ldb, 0.0, C, ldc, 0, P, ws)

    m, n, k = 6, 10, 8
    # A^T is k x m: lda must be >= m (not k); B^T is n x k: ldb must be >= k (not n)
    assert f(1, 0, m, n, k, m - 1, n, n) == E.ERROR_INVALID_LD
    assert f(0, 1, m, n, k, k, k - 1, n) == E.ERROR_INVALID_LD
    assert f(1, 1, m, n, k, m, k, n - 1) == E.ERROR_INVALID_LD
    assert f(0, 0, m, n, k, k - 1, n, n) == E.ERROR_INVALID_LD
    for bad in (-1, 2):
        assert f(bad, 0, m, n, k, 16, 16, 16) == E.ERROR_INVALID_VALUE
        assert f(0, bad, m, n, k, 16, 16, 16) == E.ERROR_INVALID_VALUE
    assert f(1, 1, m, n, k, m, k, n, A=None) == E.ERROR_NULL_POINTER
    # lda = m < k and ldb = k < n are valid for the transposed forms: the call
    # gets past every argument check (no device here, or a no-op size)
    assert f(1, 1, 0, n, k, 1, k, n) == E.SUCCESS


def test_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the no-device path")
    assert hta.mi_sgemm(4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4) == hta.ERROR_DEVICE


def test_reduce_sum_argument_errors_and_queries():
    E = hta
    assert hta.mi_reduce_sum(-1, P, P, P, 4) == E.ERROR_INVALID_VALUE
    assert hta.mi_reduce_sum(10, None, P, P, 4) == E.ERROR_NULL_POINTER
    assert hta.mi_reduce_sum(10, P, None, P, 4) == E.ERROR_NULL_POINTER
    ws = hta.mi_reduce_sum_workspace_bytes(1 << 20)
    assert ws >= 4 and ws % 4 == 0
    assert hta.mi_reduce_sum(1 << 20, P, P, P, ws - 4) == E.ERROR_WORKSPACE
    assert hta.mi_reduce_sum(1 << 20, P, P, None, ws) == E.ERROR_WORKSPACE
    assert hta.mi_reduce_sum_workspace_bytes(0) == 0
    # the stated error bound grows with the work per lane and stays small
    assert hta.mi_reduce_sum_max_additions(0) == 0
    d1 = hta.mi_reduce_sum_max_additions(1)
    dbig = hta.mi_reduce_sum_max_additions(1 << 28)
    assert 0 < d1 <= dbig < 400


def test_helpers_refuse_mixed_devices():
    """The torch helpers run each call with the operands' device current and
    refuse operands on different devices (checked here with CPU and meta
    tensors: the check comes before any device use)."""
    import torch
    a = torch.empty(2, 2)
    b = torch.empty(2, 2, device="meta")
    with pytest.raises(ValueError, match="different devices"):
        hta._device_of(a, b)
    assert hta._device_of(a, None, torch.empty(3)) == torch.device("cpu")


def test_streamk_argument_errors_and_plan():
    E, f = hta, hta.mi_sgemm_streamk
    ws = hta.mi_sgemm_streamk_workspace_bytes(-1, 100, 100, 100, 0)
    assert ws > 0
    assert f(-1, 0, 0, 100, 100, 100, 1.0, P, 100, P, 100, 0.0, P, 100, -1, P, ws) == E.ERROR_INVALID_VALUE
    assert f(99, 0, 0, 100, 100, 100, 1.0, P, 100, P, 100, 0.0, P, 100, 0, P, ws) == E.ERROR_INVALID_VALUE
    assert f(-1, 0, 0, 100, 100, 100, 1.0, P, 99, P, 100, 0.0, P, 100, 0, P, ws) == E.ERROR_INVALID_LD
    assert f(-1, 0, 0, 100, 100, 100, 1.0, P, 100, P, 100, 0.0, P, 100, 0, P, ws - 1) == E.ERROR_WORKSPACE
    assert f(-1, 0, 0, 100, 100, 100, 1.0, P, 100, P, 100, 0.0, P, 100, 0, None, ws) == E.ERROR_WORKSPACE
    assert f(-1, 0, 0, 0, 100, 100, 1.0, None, 100, None, 100, 0.0, None, 100, 0, None, 0) == E.SUCCESS
    assert hta.mi_sgemm_streamk_workspace_bytes(-1, 100, 100, 100, -1) == 0
    # the grid never exceeds the number of (tile, k step) iterations; a grid
    # that divides the tiles shares none (no workspace)
    assert hta.mi_sgemm_streamk_workspace_bytes(6, 1, 1, 5, 1000) == 0
    assert hta.mi_sgemm_streamk_workspace_bytes(6, 128, 128, 64, 4) == 0
    # 4 tiles of 64 x 64, 3 workgroups: every tile's iterations are shared
    assert hta.mi_sgemm_streamk_workspace_bytes(6, 100, 100, 100, 3) == 3 * 2 * 64 * 64 * 4 + 256
    # 16 tiles, 3 workgroups: 12 whole tiles, the last 4 shared
    assert hta.mi_sgemm_streamk_workspace_bytes(6, 256, 256, 100, 3) == 3 * 2 * 64 * 64 * 4 + 256
    # the automatic split plan picks stream-K where its model prefers it
    p = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, 1536, 1536, 4096, 0)
    assert p["stream_k_grid"] > 0 and p["workgroups"] >= p["stream_k_grid"]
    q = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, 512, 512, 262144, 0)
    assert q["stream_k_grid"] == 0 and q["splits"] == 16
    a = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK_ATOMIC, -1, 1536, 1536, 4096, 0)
    assert a["stream_k_grid"] == 0


def test_tile_choice_rules():
    """The automatic tile choice: the 16-wave 128 x 128 x 32 tile on grids of
    one or two rounds, the 8-wave 128 x 128 x 16 tile for two workgroups per
    CU from 3 rounds of 128 x 128 tiles, 64 x 64 x 32 where it quantises better, and 64 x 64 x 16
    (six workgroups per CU) when k leaves a partial 32-wide step on 8 or more
    rounds of 64 x 64 tiles, in its four-buffer form (four per CU) from
    k = 848 on."""
    def tile(m, n, k):
        p = hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, -1, m, n, k, 0)
        return p["tile_m"], p["tile_n"], p["tile_k"], p["threads"]
    assert tile(2048, 2048, 2048) == (128, 128, 32, 1024)      # one round of 128 x 128
    assert tile(2048, 4096, 2048) == (128, 128, 32, 1024)      # two rounds
    assert tile(3072, 4096, 4096) == (128, 128, 16, 512)       # three: two per CU, 4 x 2 waves
    assert tile(4096, 4096, 4096) == (128, 128, 16, 512)
    assert tile(8192, 8192, 8192) == (128, 128, 16, 512)
    assert tile(12288, 12288, 4096) == (128, 128, 16, 512)
    assert tile(3072, 3072, 3072) == (64, 64, 32, 256)
    assert tile(3001, 4997, 1023) == (64, 64, 16, 256)         # partial k step, 3713 tiles
    assert tile(3001, 4997, 1024) == (64, 64, 32, 256)         # whole k steps
    assert tile(1000, 1000, 1000) == (64, 64, 32, 256)         # short grid
    config = lambda m, n, k: hta.mi_sgemm_get_plan(hta.KERNEL_MFMA, -1, m, n, k, 0)["config"]
    assert config(3001, 4997, 1023) == 13                      # four buffers, long k
    assert config(2500, 6000, 847) == 12 and config(2500, 6000, 849) == 13
    assert config(2500, 6000, 777) == 12                       # three buffers, short k
    # stream-K on the 64 x 64 x 32 tile with one workgroup per CU, for small
    # grids with 1024 <= k <= 2048
    def sk(m, n, k):
        q = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, m, n, k, 0)
        return q["config"], q["splits"], q["stream_k_grid"]
    assert sk(768, 768, 1024) == (6, 1, 256)
    assert sk(1536, 1536, 1024) == (6, 1, 256)
    assert sk(1536, 1536, 2048) == (6, 1, 256)                 # over a 128 x 128 stream-K plan
    assert sk(2304, 2304, 1024) == (6, 1, 256)
    assert sk(1280, 1280, 1024) == (8, 1, 0)                   # the single pass stays
    assert sk(1536, 1536, 4096) == (9, 1, 256)                 # k above the range
    assert sk(768, 768, 512) == (6, 1, 0)                      # k below it: single pass
    # the split-K entry's single-slice plans use the same choice
    p = hta.mi_sgemm_get_plan(hta.KERNEL_SPLITK, -1, 8192, 8192, 8192, 0)
    assert p["splits"] == 1 and (p["tile_m"], p["tile_k"], p["threads"]) == (128, 16, 512)


@pytest.mark.parametrize("helper", ["sgemm", "sgemm_valu", "sgemm_splitk", "sgemm_streamk",
                                    "sgemm_splitk_atomic"])
def test_helpers_refuse_host_operands(helper):
    """The torch helpers take device tensors only: a numpy array or a CPU
    tensor is refused before any device call."""
    import numpy as np
    import torch
    fn = getattr(hta, helper)
    with pytest.raises(TypeError, match="torch.Tensor"):
        fn(np.zeros((2, 2), np.float32), torch.empty(2, 2))
    with pytest.raises(ValueError, match="device tensor"):
        fn(torch.empty(2, 2), torch.empty(2, 2))


def test_reduce_sum_refuses_host_input():
    import torch
    with pytest.raises(TypeError, match="float32 device tensor"):
        hta.reduce_sum(torch.ones(8))
    with pytest.raises(TypeError, match="float32 device tensor"):
        hta.reduce_sum([1.0, 2.0])

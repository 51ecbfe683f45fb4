"""Python binding of libmi_sgemm (single-precision GEMM for MI355X / gfx950).

Thin ctypes layer over the C ABI declared in ``include/mi_sgemm.h``: the
functions named like the C entry points (``mi_sgemm``, ``mi_sgemm_valu``,
``mi_sgemm_splitk``, ...) take the same arguments (device pointers as
integers, the stream as an integer handle); the ``sgemm*`` helpers marshal
torch tensors to them.  Every step of the computation runs in the library's
HIP kernels; there is no fallback path.  Importing raises ImportError when the
library has not been built (``python hpc_tiling_amd/build.py``).

torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

__all__ = [
    "LIB_PATH", "lib", "MiSgemmError", "Plan",
    "mi_sgemm", "mi_sgemm_valu", "mi_sgemm_splitk", "mi_sgemm_splitk_workspace_bytes",
    "mi_status_string", "mi_sgemm_get_plan", "mi_sgemm_config_count", "mi_sgemm_with_config",
    "mi_sgemm_splitk_with_config", "mi_sgemm_splitk_with_config_workspace_bytes",
    "mi_sgemm_splitk_atomic", "mi_reduce_sum", "mi_reduce_sum_workspace_bytes",
    "mi_reduce_sum_max_additions", "mi_sgemm_ex", "mi_sgemm_splitk_ex", "mi_sgemm_streamk",
    "mi_sgemm_streamk_workspace_bytes", "mi_sgemm_splitk_combine", "mi_clock_probe",
    "mi_sgemm_with_order", "mi_sgemm_splitk_noalloc", "mi_fma_rate_probe",
    "sgemm", "sgemm_streamk", "streamk_workspace", "sgemm_valu", "sgemm_splitk", "sgemm_splitk_atomic", "splitk_workspace", "splitk_combine", "reduce_sum", "ClockProbe",
    "KERNEL_MFMA", "KERNEL_VALU", "KERNEL_SPLITK", "KERNEL_SPLITK_ATOMIC", "EXPORTED_SYMBOLS",
    "OP_N", "OP_T",
]

LIB_PATH = Path(__file__).resolve().parent / "libmi_sgemm.so"

SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_INVALID_LD = 2
ERROR_NULL_POINTER = 3
ERROR_WORKSPACE = 4
ERROR_LAUNCH = 5
ERROR_DEVICE = 6
ERROR_SCRATCH_LIMIT = 7
NOALLOC_SCRATCH_BYTES = 64 << 20

KERNEL_MFMA = 0
KERNEL_VALU = 1
KERNEL_SPLITK = 2
KERNEL_SPLITK_ATOMIC = 3

OP_N = 0  # operand as given
OP_T = 1  # operand given transposed (A stored k x m, B stored n x k)

EXPORTED_SYMBOLS = (
    "mi_sgemm", "mi_sgemm_valu", "mi_sgemm_splitk_workspace_bytes", "mi_sgemm_splitk",
    "mi_status_string", "mi_sgemm_get_plan", "mi_sgemm_config_count", "mi_sgemm_with_config",
    "mi_sgemm_splitk_with_config", "mi_sgemm_splitk_with_config_workspace_bytes",
    "mi_sgemm_splitk_atomic", "mi_reduce_sum", "mi_reduce_sum_workspace_bytes",
    "mi_reduce_sum_max_additions", "mi_sgemm_ex", "mi_sgemm_splitk_ex", "mi_sgemm_streamk",
    "mi_sgemm_streamk_workspace_bytes", "mi_sgemm_splitk_combine", "mi_clock_probe",
    "mi_sgemm_with_order", "mi_sgemm_splitk_noalloc", "mi_fma_rate_probe",
)

if not LIB_PATH.exists():
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python hpc_tiling_amd/build.py` "
        "(the HIP library is required; there is no other implementation)")

# torch bundles its own HIP runtime under the same SONAME (libamdhip64.so.7).
# Loading torch first makes the library bind to that runtime instead of
# pulling a second copy into the process (device pointers and streams are only
# valid in the runtime that created them).
try:
    import torch as _torch  # noqa: F401
except ImportError:  # pragma: no cover - C callers without torch
    _torch = None

lib = ctypes.CDLL(str(LIB_PATH))

_i, _f, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_GEMM_ARGS = [_i, _i, _i, _f, _vp, _i, _vp, _i, _f, _vp, _i]


class Plan(ctypes.Structure):
    """Mirror of struct mi_sgemm_plan."""
    _fields_ = [
        ("kernel", _i), ("config", _i),
        ("tile_m", _i), ("tile_n", _i), ("tile_k", _i),
        ("micro_m", _i), ("micro_n", _i), ("threads", _i),
        ("tiles_m", _i), ("tiles_n", _i), ("workgroups", ctypes.c_longlong),
        ("splits", _i), ("k_per_split", _i), ("big_iterations", _i),
        ("small_iterations", _i), ("fma_per_small_iteration", _i),
        ("outputs_per_thread", _i), ("a_elements_per_big_iteration", _i),
        ("b_elements_per_big_iteration", _i), ("group_m", _i), ("vector_loads", _i),
        ("workspace_bytes", _sz), ("stream_k_grid", _i),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


lib.mi_sgemm.argtypes = _GEMM_ARGS + [_vp]
lib.mi_sgemm.restype = _i
lib.mi_sgemm_valu.argtypes = _GEMM_ARGS + [_vp]
lib.mi_sgemm_valu.restype = _i
lib.mi_sgemm_ex.argtypes = [_i, _i] + _GEMM_ARGS + [_vp]
lib.mi_sgemm_ex.restype = _i
lib.mi_sgemm_with_config.argtypes = [_i, _i, _i, _i] + _GEMM_ARGS + [_vp]
lib.mi_sgemm_with_config.restype = _i
lib.mi_sgemm_with_order.argtypes = [_i, _i, _i, _i, _i] + _GEMM_ARGS + [_vp]
lib.mi_sgemm_with_order.restype = _i
lib.mi_sgemm_splitk_workspace_bytes.argtypes = [_i, _i, _i, _i]
lib.mi_sgemm_splitk_workspace_bytes.restype = _sz
lib.mi_sgemm_splitk.argtypes = _GEMM_ARGS + [_i, _vp, _sz, _vp]
lib.mi_sgemm_splitk.restype = _i
lib.mi_sgemm_splitk_ex.argtypes = [_i, _i] + _GEMM_ARGS + [_i, _vp, _sz, _vp]
lib.mi_sgemm_splitk_ex.restype = _i
lib.mi_sgemm_splitk_noalloc.argtypes = [_i, _i] + _GEMM_ARGS + [_i, _vp]
lib.mi_sgemm_splitk_noalloc.restype = _i
lib.mi_sgemm_splitk_with_config.argtypes = [_i, _i, _i] + _GEMM_ARGS + [_i, _vp, _sz, _vp]
lib.mi_sgemm_splitk_with_config.restype = _i
lib.mi_sgemm_splitk_with_config_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
lib.mi_sgemm_splitk_with_config_workspace_bytes.restype = _sz
lib.mi_sgemm_streamk.argtypes = [_i, _i, _i] + _GEMM_ARGS + [_i, _vp, _sz, _vp]
lib.mi_sgemm_streamk.restype = _i
lib.mi_sgemm_streamk_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
lib.mi_sgemm_streamk_workspace_bytes.restype = _sz
lib.mi_sgemm_splitk_combine.argtypes = [_i, _i, _i, _vp, ctypes.c_longlong, _f, _f, _vp, _i, _vp]
lib.mi_sgemm_splitk_combine.restype = _i
lib.mi_fma_rate_probe.argtypes = [_i, _vp, _i, _i, _vp]
lib.mi_fma_rate_probe.restype = _i
lib.mi_clock_probe.argtypes = [_vp, _i, _i, ctypes.POINTER(_i), _vp]
lib.mi_clock_probe.restype = _i
lib.mi_sgemm_splitk_atomic.argtypes = _GEMM_ARGS + [_i, _vp]
lib.mi_sgemm_splitk_atomic.restype = _i
lib.mi_reduce_sum.argtypes = [ctypes.c_longlong, _vp, _vp, _vp, _sz, _vp]
lib.mi_reduce_sum.restype = _i
lib.mi_reduce_sum_workspace_bytes.argtypes = [ctypes.c_longlong]
lib.mi_reduce_sum_workspace_bytes.restype = _sz
lib.mi_reduce_sum_max_additions.argtypes = [ctypes.c_longlong]
lib.mi_reduce_sum_max_additions.restype = ctypes.c_longlong
lib.mi_status_string.argtypes = [_i]
lib.mi_status_string.restype = ctypes.c_char_p
lib.mi_sgemm_get_plan.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(Plan)]
lib.mi_sgemm_get_plan.restype = _i
lib.mi_sgemm_config_count.argtypes = [_i]
lib.mi_sgemm_config_count.restype = _i


class MiSgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mi_status_string(status)} (status {status})")


# ---------------------------------------------------------------------------
# C entry points, same names and arguments
# ---------------------------------------------------------------------------
def mi_sgemm(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return lib.mi_sgemm(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def mi_sgemm_valu(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    return lib.mi_sgemm_valu(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def mi_sgemm_ex(trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                stream=None) -> int:
    return lib.mi_sgemm_ex(trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                           stream)


def mi_sgemm_with_config(kernel, config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb,
                         beta, C, ldc, stream=None) -> int:
    return lib.mi_sgemm_with_config(kernel, config, trans_a, trans_b, m, n, k, alpha, A, lda,
                                    B, ldb, beta, C, ldc, stream)


def mi_sgemm_with_order(config, xcd_remap, group_m, trans_a, trans_b, m, n, k, alpha, A, lda, B,
                        ldb, beta, C, ldc, stream=None) -> int:
    return lib.mi_sgemm_with_order(config, xcd_remap, group_m, trans_a, trans_b, m, n, k, alpha,
                                   A, lda, B, ldb, beta, C, ldc, stream)


def mi_sgemm_splitk_workspace_bytes(m, n, k, splits=0) -> int:
    return lib.mi_sgemm_splitk_workspace_bytes(m, n, k, splits)


def mi_sgemm_splitk(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits, ws, ws_bytes,
                    stream=None) -> int:
    return lib.mi_sgemm_splitk(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits, ws,
                               ws_bytes, stream)


def mi_sgemm_splitk_ex(trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                       ws, ws_bytes, stream=None) -> int:
    return lib.mi_sgemm_splitk_ex(trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C,
                                  ldc, splits, ws, ws_bytes, stream)


def mi_sgemm_splitk_noalloc(trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                            splits, stream=None) -> int:
    return lib.mi_sgemm_splitk_noalloc(trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C,
                                       ldc, splits, stream)


def mi_sgemm_splitk_with_config(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta,
                                C, ldc, splits, ws, ws_bytes, stream=None) -> int:
    return lib.mi_sgemm_splitk_with_config(config, trans_a, trans_b, m, n, k, alpha, A, lda, B,
                                           ldb, beta, C, ldc, splits, ws, ws_bytes, stream)


def mi_sgemm_splitk_with_config_workspace_bytes(config, m, n, k, splits=0) -> int:
    return lib.mi_sgemm_splitk_with_config_workspace_bytes(config, m, n, k, splits)


def mi_sgemm_streamk(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                     grid, ws, ws_bytes, stream=None) -> int:
    return lib.mi_sgemm_streamk(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta,
                                C, ldc, grid, ws, ws_bytes, stream)


def mi_sgemm_streamk_workspace_bytes(config, m, n, k, grid=0) -> int:
    return lib.mi_sgemm_streamk_workspace_bytes(config, m, n, k, grid)


def mi_sgemm_splitk_atomic(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits=0,
                           stream=None) -> int:
    return lib.mi_sgemm_splitk_atomic(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                                      stream)


def mi_sgemm_splitk_combine(m, n, splits, ws, slice, alpha, beta, C, ldc, stream=None) -> int:
    return lib.mi_sgemm_splitk_combine(m, n, splits, ws, slice, alpha, beta, C, ldc, stream)


def mi_fma_rate_probe(loop, out, workgroups, iters, stream=None) -> int:
    return lib.mi_fma_rate_probe(loop, out, workgroups, iters, stream)


def mi_clock_probe(ticks, workgroups, spin_us, ref_khz, stream=None) -> int:
    """ref_khz: a ctypes.c_int (passed by reference)."""
    return lib.mi_clock_probe(ticks, workgroups, spin_us, ctypes.byref(ref_khz), stream)


def mi_reduce_sum(n, x, out, ws, ws_bytes, stream=None) -> int:
    return lib.mi_reduce_sum(n, x, out, ws, ws_bytes, stream)


def mi_reduce_sum_workspace_bytes(n) -> int:
    return lib.mi_reduce_sum_workspace_bytes(n)


def mi_reduce_sum_max_additions(n) -> int:
    return lib.mi_reduce_sum_max_additions(n)


def mi_status_string(status: int) -> str:
    return lib.mi_status_string(status).decode()


def mi_sgemm_get_plan(kernel, config, m, n, k, splits=0) -> dict:
    p = Plan()
    st = lib.mi_sgemm_get_plan(kernel, config, m, n, k, splits, ctypes.byref(p))
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_get_plan")
    return p.as_dict()


def mi_sgemm_config_count(kernel) -> int:
    return lib.mi_sgemm_config_count(kernel)


# ---------------------------------------------------------------------------
# torch tensor helpers
# ---------------------------------------------------------------------------
def _mat(t, name):
    """(pointer, ld, transposed, rows, cols, device index) of a 2-D float32
    device tensor stored row-major (unit column stride; ld = row stride) or
    column-major (unit row stride, i.e. the transpose of a row-major matrix;
    ld = column stride).  Each tensor attribute is read once: these checks
    sit in front of every call."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    dev = t.get_device()
    if dev < 0:
        raise ValueError(f"{name} must be a device tensor")
    shape = t.shape
    if len(shape) != 2:
        raise ValueError(f"{name} must be 2-D")
    r, c = shape
    s0, s1 = t.stride()
    if c <= 1 or s1 == 1:
        ld = max(s0, c, 1) if r > 1 else max(c, 1)
        return t.data_ptr(), ld, OP_N, r, c, dev
    if r <= 1 or s0 == 1:
        ld = max(s1, r, 1) if c > 1 else max(r, 1)
        return t.data_ptr(), ld, OP_T, r, c, dev
    raise ValueError(f"{name} must be row-major or column-major (one unit stride)")


class _Unchanged:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


_UNCHANGED = _Unchanged()


def _stream(stream, device):
    """The HIP stream handle: `stream` (a torch stream or a raw handle), else
    the current stream of device index `device`."""
    import torch
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tensor_device(t, name):
    """Device index of tensor `t` (checked again, with the other properties,
    when its layout is read)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    dev = t.get_device()
    if dev < 0:
        raise ValueError(f"{name} must be a device tensor")
    return dev


def _on_stream(stream, device):
    """A context in which `stream` (None: the current stream, nothing
    changes) is torch's current stream on device index `device`.  The helpers
    allocate C and workspaces inside it, so the caching allocator ties those
    blocks to the stream the kernels run on: a block freed on return is
    handed out again only to work ordered after those kernels on that
    stream."""
    import torch
    if stream is None:
        return _UNCHANGED
    if not isinstance(stream, torch.cuda.Stream):
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        if handle == torch._C._cuda_getCurrentRawStream(device):
            return _UNCHANGED
        stream = torch.cuda.ExternalStream(handle, device=device)
    return torch.cuda.stream(stream)


def _device_of(*tensors):
    """The one device all given tensors (None skipped) live on; tensors on
    different devices are refused."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"tensors are on different devices: {sorted(str(d) for d in devs)}")
    return devs.pop()


def _current(dev):
    """A context with device index `dev` current: the library launches on the
    current device.  The device is switched only when it differs."""
    import torch
    if torch.cuda.current_device() == dev:
        return _UNCHANGED
    return torch.cuda.device(dev)


def _same_device(dev, *tensors):
    """Refuse tensors (None skipped) that are not on device index `dev`."""
    for t in tensors:
        if t is not None and t.get_device() != dev:
            raise ValueError(f"tensors are on different devices: cuda:{dev} and {t.device}")


def _mats(A, B, C, beta):
    """Layouts of A (m x k), B (k x n) and C (m x n, allocated when None):
    (A's, B's, C's (pointer, ld, transposed), m, n, k, C, device index)."""
    import torch
    pa, lda, ta, m, k, da = _mat(A, "A")
    pb, ldb, tb, k2, n, db = _mat(B, "B")
    if k2 != k:
        raise ValueError(f"inner sizes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if C is None:
        if beta != 0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((m, n), dtype=torch.float32, device=A.device)
    pc, ldc, tc, mc, nc, dc = _mat(C, "C")
    if mc != m or nc != n:
        raise ValueError(f"C is {tuple(C.shape)}, expected {(m, n)}")
    if not da == db == dc:
        _same_device(da, A, B, C)
    return (pa, lda, ta), (pb, ldb, tb), (pc, ldc, tc), m, n, k, C, da


def _prepare(A, B, C, beta):
    """Row-major A, B and C (the VALU and atomic paths)."""
    a, b, c, m, n, k, C, dev = _mats(A, B, C, beta)
    for (_, _, trans), name in ((a, "A"), (b, "B"), (c, "C")):
        if trans != OP_N:
            raise ValueError(f"{name} must be row-major (unit column stride)")
    return m, n, k, a[0], a[1], b[0], b[1], C, c[0], c[1], dev


def _prepare_ex(A, B, C, beta):
    """Operands in either storage order.  A column-major C is written as its
    row-major transpose: C^T = op(B)^T op(A)^T, i.e. the call with A and B
    swapped, each with its transpose flag flipped."""
    (pa, lda, ta), (pb, ldb, tb), (pc, ldc, tc), m, n, k, C, dev = _mats(A, B, C, beta)
    if tc == OP_N:
        return (ta, tb, m, n, k, pa, lda, pb, ldb), C, pc, ldc, dev
    return (1 - tb, 1 - ta, n, m, k, pb, ldb, pa, lda), C, pc, ldc, dev


def sgemm(A, B, C=None, alpha=1.0, beta=0.0, stream=None, config=None, order=None):
    """C <- alpha * A @ B + beta * C on the matrix cores; returns C.
    A (m x k), B (k x n), C (m x n): float32 device tensors, each row-major
    or column-major (a transposed view such as ``X.t()`` is passed as the
    transposed operand, without a copy).  `order` = (xcd_remap, group_m)
    forces the workgroup order (mi_sgemm_with_order)."""
    dev = _tensor_device(A, "A")
    with _current(dev), _on_stream(stream, dev):
        (ta, tb, m, n, k, pa, lda, pb, ldb), C, pc, ldc, dev = _prepare_ex(A, B, C, beta)
        s = _stream(None, dev)
        if order is not None:
            st = lib.mi_sgemm_with_order(-1 if config is None else config, order[0], order[1],
                                         ta, tb, m, n, k, alpha, pa, lda, pb, ldb, beta, pc,
                                         ldc, s)
        elif config is None:
            st = lib.mi_sgemm_ex(ta, tb, m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc, s)
        else:
            st = lib.mi_sgemm_with_config(KERNEL_MFMA, config, ta, tb, m, n, k, alpha, pa, lda,
                                          pb, ldb, beta, pc, ldc, s)
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_ex")
    return C


def sgemm_valu(A, B, C=None, alpha=1.0, beta=0.0, stream=None, config=None):
    """Same as sgemm (row-major operands only), on the register-tiled VALU
    kernel; `config` forces its configuration (0: one k group, 1: two)."""
    dev = _tensor_device(A, "A")
    with _current(dev), _on_stream(stream, dev):
        m, n, k, pa, lda, pb, ldb, C, pc, ldc, dev = _prepare(A, B, C, beta)
        s = _stream(None, dev)
        if config is None:
            st = lib.mi_sgemm_valu(m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc, s)
        else:
            st = lib.mi_sgemm_with_config(KERNEL_VALU, config, 0, 0, m, n, k, alpha, pa, lda,
                                          pb, ldb, beta, pc, ldc, s)
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_valu")
    return C


def splitk_workspace(m, n, k, splits=0, device="cuda", config=None):
    """A device workspace tensor large enough for mi_sgemm_splitk (or, with
    `config`, for mi_sgemm_splitk_with_config)."""
    import torch
    if config is None:
        nbytes = mi_sgemm_splitk_workspace_bytes(m, n, k, splits)
    else:
        nbytes = mi_sgemm_splitk_with_config_workspace_bytes(config, m, n, k, splits)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def sgemm_splitk(A, B, C=None, alpha=1.0, beta=0.0, splits=0, workspace=None, stream=None,
                 config=None):
    """Same as sgemm with the k range split into slices; `workspace` is a
    device tensor of at least mi_sgemm_splitk_workspace_bytes bytes (allocated
    here when None).  `config` forces the partial kernel's tile configuration."""
    dev = _tensor_device(A, "A")
    with _current(dev), _on_stream(stream, dev):
        (ta, tb, m, n, k, pa, lda, pb, ldb), C, pc, ldc, dev = _prepare_ex(A, B, C, beta)
        if workspace is None:
            workspace = splitk_workspace(m, n, k, splits, device=A.device, config=config)
        _same_device(dev, workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
        s = _stream(None, dev)
        if config is None:
            st = lib.mi_sgemm_splitk_ex(ta, tb, m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc,
                                        splits, workspace.data_ptr(), ws_bytes, s)
        else:
            st = lib.mi_sgemm_splitk_with_config(config, ta, tb, m, n, k, alpha, pa, lda, pb,
                                                 ldb, beta, pc, ldc, splits,
                                                 workspace.data_ptr(), ws_bytes, s)
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_splitk_ex")
    return C


def streamk_workspace(m, n, k, grid=0, device="cuda", config=-1):
    """A device workspace tensor large enough for mi_sgemm_streamk."""
    import torch
    nbytes = mi_sgemm_streamk_workspace_bytes(config, m, n, k, grid)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def sgemm_streamk(A, B, C=None, alpha=1.0, beta=0.0, grid=0, workspace=None, stream=None,
                  config=-1):
    """Same as sgemm on a forced stream-K schedule (`grid` workgroups, 0 for
    one per resident slot of every CU); `workspace` as streamk_workspace."""
    dev = _tensor_device(A, "A")
    with _current(dev), _on_stream(stream, dev):
        (ta, tb, m, n, k, pa, lda, pb, ldb), C, pc, ldc, dev = _prepare_ex(A, B, C, beta)
        if workspace is None:
            workspace = streamk_workspace(m, n, k, grid, device=A.device, config=config)
        _same_device(dev, workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
        st = lib.mi_sgemm_streamk(config, ta, tb, m, n, k, alpha, pa, lda, pb, ldb, beta, pc,
                                  ldc, grid, workspace.data_ptr(), ws_bytes, _stream(None, dev))
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_streamk")
    return C


def sgemm_splitk_atomic(A, B, C=None, alpha=1.0, beta=0.0, splits=0, stream=None):
    """Split-K with atomic accumulation into C (row-major operands; no
    workspace; not bitwise reproducible run to run)."""
    dev = _tensor_device(A, "A")
    with _current(dev), _on_stream(stream, dev):
        m, n, k, pa, lda, pb, ldb, C, pc, ldc, dev = _prepare(A, B, C, beta)
        st = lib.mi_sgemm_splitk_atomic(m, n, k, alpha, pa, lda, pb, ldb, beta, pc, ldc, splits,
                                        _stream(None, dev))
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_splitk_atomic")
    return C


def splitk_combine(parts, C, alpha=1.0, beta=0.0, stream=None):
    """C <- alpha * parts.sum(0) + beta * C through mi_sgemm_splitk_combine.
    parts: float32 device tensor (S, m, n) or (S, slice) with contiguous
    slices (16-byte aligned, slice a multiple of 4 and >= m*n rounded up to
    4); C: m x n row-major float32 device tensor (row stride = ldc)."""
    import torch
    if not isinstance(parts, torch.Tensor) or parts.dtype != torch.float32 or not parts.is_cuda:
        raise TypeError("parts must be a float32 device tensor")
    S = parts.shape[0]
    slice_ = parts.stride(0) if S > 1 else max(parts[0].numel(), 4)
    dev = parts.get_device()
    pc, ldc, tc, m, n, dc = _mat(C, "C")
    if tc != OP_N:
        raise ValueError("C must be row-major (unit column stride)")
    _same_device(dev, C)
    with _current(dev):
        st = lib.mi_sgemm_splitk_combine(m, n, S, parts.data_ptr(), slice_, alpha, beta, pc,
                                         ldc, _stream(stream, dev))
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_sgemm_splitk_combine")
    return C


class ClockProbe:
    """Core clock measured on the GPU in stream order (mi_clock_probe): call
    launch() where the clock is wanted, and mhz() after synchronising."""

    def __init__(self, workgroups=8, spin_us=20, device=None):
        import torch
        self.workgroups, self.spin_us = workgroups, spin_us
        self.ticks = torch.zeros(4 * workgroups, dtype=torch.int64, device=device or "cuda")
        self.ref_khz = ctypes.c_int(0)

    def launch(self, stream=None):
        dev = self.ticks.get_device()
        with _current(dev):
            st = lib.mi_clock_probe(self.ticks.data_ptr(), self.workgroups, self.spin_us,
                                    ctypes.byref(self.ref_khz), _stream(stream, dev))
        if st != SUCCESS:
            raise MiSgemmError(st, "mi_clock_probe")

    def mhz(self):
        """Per-workgroup clocks in MHz of the last launch (host list)."""
        t = self.ticks.cpu().tolist()
        out = []
        for w in range(self.workgroups):
            c0, r0, c1, r1 = t[4 * w:4 * w + 4]
            out.append((c1 - c0) / max(r1 - r0, 1) * self.ref_khz.value / 1e3)
        return out


def reduce_sum(x, out=None, workspace=None, stream=None):
    """Sum of a 1-D float32 device tensor (contiguous); returns a 1-element
    device tensor."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda:
        raise TypeError("x must be a float32 device tensor")
    if x.dim() != 1 or (x.numel() > 1 and x.stride(0) != 1):
        raise ValueError("x must be 1-D and contiguous")
    n = x.numel()
    dev = x.get_device()
    with _current(dev), _on_stream(stream, dev):
        if out is None:
            out = torch.empty(1, dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(mi_reduce_sum_workspace_bytes(n), 4), dtype=torch.uint8,
                                    device=x.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        _same_device(dev, out, workspace)
        st = lib.mi_reduce_sum(n, x.data_ptr() if n else None, out.data_ptr(),
                               workspace.data_ptr(), ws_bytes, _stream(None, dev))
    if st != SUCCESS:
        raise MiSgemmError(st, "mi_reduce_sum")
    return out

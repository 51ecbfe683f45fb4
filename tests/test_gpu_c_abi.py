"""The C ABI from plain C: tests/c_abi/abi_demo (built with gcc by
hpc_tiling_amd/build.py) allocates device memory with the HIP runtime, calls
mi_sgemm, mi_sgemm_ex (both operands transposed), mi_sgemm_splitk,
mi_sgemm_splitk_noalloc (twice) and mi_reduce_sum on integer-valued data,
checks each result exactly against 64-bit integer sums, and checks three
argument errors.  It runs as a child
process with no Python or torch inside."""
import subprocess
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

DEMO = Path(__file__).resolve().parent / "c_abi" / "abi_demo"


def test_c_program_through_the_abi():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not DEMO.exists():
        pytest.fail(f"{DEMO} is missing: build it with `python hpc_tiling_amd/build.py`")
    print("[case] c abi demo", flush=True)
    res = subprocess.run([str(DEMO)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi demo ok" in res.stdout

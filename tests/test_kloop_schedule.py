"""The k-step schedule of the matrix-core kernel, checked on the host.

tests/kloop/kloop_sim.cpp replays the kernel's loop over the k steps of a
tile (prologue, steady loop, deciding loop, fixed or decided tail) with the
schedule functions the kernel includes (hpc_tiling_amd/csrc/kloop.hpp), for
1 to 64 steps on rings of 2 to 4 buffers, with direct loads off, every step
whole, or a partial last step (loaded directly with its k tail masked when
direct loads are on).  It checks that every step runs exactly once on its
ring position, every tile is loaded once (directly when it is a whole k step,
or the partial step with direct loads on), and no tile is read before a
barrier has waited for it.

The replay is pinned by mistakes planted in copies of the header: each one
must make it fail.  "alias_negative_whole_steps" is the kind of key aliasing
that once made the kernel skip k steps when direct loads were off.
"""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "hpc_tiling_amd" / "csrc" / "kloop.hpp"
SIM = Path(__file__).resolve().parent / "kloop" / "kloop_sim.cpp"

# (name, exact text in kloop.hpp, replacement)
MUTANTS = [
    ("alias_negative_whole_steps", "if (ns >= 3 && nd >= 0) k.tail = tail_index(r, nd);",
     "if (ns >= 3) k.tail = tail_index(r, nd < 0 ? r - 1 : nd);"),
    ("tail_ignores_whole_steps",
     "if (kTailSequences[i].r == r && kTailSequences[i].nd == nd) return i;",
     "if (kTailSequences[i].r == r) return i;"),
    ("steady_one_round_long", "k.steady_end = ns * ceil_pos(ndirect - (ns - 1 + d), ns);",
     "k.steady_end = ns * ceil_pos(ndirect - (ns - 1 + d) + 1, ns);"),
    ("tail_one_step_long",
     "k.auto_end = k.steady_end + ns * ceil_pos(nsteps - kTailMax - k.steady_end, ns);",
     "k.auto_end = k.steady_end + ns * ceil_pos(nsteps - kTailMax - 1 - k.steady_end, ns);"),
    ("direct_partial_step", "(t < ndirect ? kLoadDirect : kLoadRegs)",
     "(t <= ndirect ? kLoadDirect : kLoadRegs)"),
    ("load_one_past_end", "return t >= nsteps ? kLoadNone", "return t > nsteps ? kLoadNone"),
    ("masked_load_with_direct_off", "return load == kLoadDirect || (load == kLoadRegs && direct_on);",
     "return load == kLoadDirect || load == kLoadRegs;"),
    ("in_flight_on_three_buffers", "return ns == 4 && loads_directly(load, direct_on);",
     "return ns >= 3 && loads_directly(load, direct_on);"),
]


def _cxx():
    for name in ("g++", "c++", "clang++"):
        if shutil.which(name):
            return name
    pytest.skip("no host C++ compiler")


def _build_and_run(include_dir: Path, exe: Path):
    subprocess.run([_cxx(), "-std=c++17", "-O1", "-Wall", f"-I{include_dir}", str(SIM),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)


def test_schedule_replay(tmp_path):
    res = _build_and_run(HEADER.parent, tmp_path / "kloop_sim")
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("0 failed"), res.stdout


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_replay(tmp_path, name, old, new):
    text = HEADER.read_text()
    assert text.count(old) == 1, f"mutant {name}: text not found once in kloop.hpp"
    (tmp_path / "kloop.hpp").write_text(text.replace(old, new))
    res = _build_and_run(tmp_path, tmp_path / "kloop_sim")
    assert res.returncode == 1, f"mutant {name} was not caught:\n{res.stdout}"
    assert "FAIL" in res.stdout

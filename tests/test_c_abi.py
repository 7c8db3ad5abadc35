"""The library driven from plain C (tests/c_abi_example.c, built by build()): device
memory from the HIP runtime, plain pointers, no Python between the caller and the ABI.
The program checks hand-derived results: a selection with sinks, window, one draft pick
and a position-ordered tie; sparse and dense attention over all-zero keys (O = mean of
the attended V rows, LSE = ln of their count); a rejected argument."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi_example")


def _run():
    assert os.path.exists(BIN), "tests/c_abi_example is built by __graft_entry__.build()"
    return subprocess.run([BIN], capture_output=True, text=True, timeout=120)


def test_c_program_links_against_the_library():
    """The program loads libdustin.so through its rpath; without a GPU it stops at the
    device count (exit 3), with one it runs every check (exit 0)."""
    r = _run()
    assert r.returncode in (0, 3), r.stdout + r.stderr


@pytest.mark.gpu
def test_c_program_checks_pass():
    r = _run()
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "c abi example ok" in r.stdout, r.stdout + r.stderr

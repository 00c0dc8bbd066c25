"""The library used from C++ alone: tests/c_abi_check.cpp allocates with
hipMalloc, calls block_attend, lmhead_confidence and unmask_select through
include/sprint.h and checks closed-form results (uniform attention over equal
keys gives the mean of V; an all-zero LM head gives confidence 1/V and argmax
0; one unmask step accepts ceil(m / steps_left) positions).  The program is
linked by the package's build step."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi_check")


@pytest.mark.gpu
def test_c_program_through_the_abi():
    assert os.path.exists(EXE), "tests/c_abi_check is missing: run python -m sparse_prefix_kv_amd.build"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=90)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout

"""The C ABI used from plain C (no torch): runs the program built from
tests/c_abi/route_smoke.c by the library build."""
import os
import subprocess

import pytest

from tests.gpu_common import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]
BIN = os.path.join(os.path.dirname(__file__), "c_abi", "route_smoke.bin")


def test_plain_c_program_runs_the_path():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built; run `python expert_grouping_dispatch_amd/build_lib.py`")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi ok" in r.stdout

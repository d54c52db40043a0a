"""The C ABI from a C++ caller with no Python in between: tests/c/abi_parity
(built by build()) fills device buffers with hipMalloc/hipMemcpy, calls
gdn_spec_decode_update and checks the result against the C oracle.  It runs
as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_parity")


def test_c_abi_parity():
    assert os.path.exists(BIN), "tests/c/abi_parity is not built (run build())"
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ABI_PARITY ok" in res.stdout

"""The library through its C ABI alone: a plain C program (tests/c_abi) that
allocates with the HIP runtime, quantizes and multiplies through include/fp4.h
and checks the results against the C oracle."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_consumer")


def test_plain_c_consumer():
    assert os.path.exists(BIN), "tests/c_abi/abi_consumer is not built (run __graft_entry__.build())"
    say("plain C consumer")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert "abi consumer ok" in r.stdout

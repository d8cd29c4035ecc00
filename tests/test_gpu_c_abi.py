"""The C ABI from C++ with no Python in between (needs an MI355X).

tests/c_abi/pkv_c_abi_test.cpp allocates with hipMalloc, calls pkv_decode,
pkv_decode_noalloc and the host checks, and compares against closed forms
(equal keys give the mean of V; one token gives its V row bit for bit) on
NaN-poisoned pools behind shuffled block tables. The program is built with the
library (__graft_entry__.build()); this test runs it and requires every case
to pass.
"""

from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "pkv_c_abi_test")


def test_c_abi_program_passes():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built: run __graft_entry__.build() first")
    print("[gpu] C ABI program", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all passed" in res.stdout

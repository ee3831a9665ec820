"""The whole path through the C ABI from a native program: no Python binding,
no torch (tests/native/abi_check.cpp, built by __graft_entry__.build()).

The program checks, in each precision, that the dense entry point equals the
sparse kernel given every block bit for bit, that a constant V comes out of
the whole path as that constant (within one bf16 ulp), and that argument
errors come back as status codes.
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_check")


@pytest.mark.parametrize("precision", ["bf16", "mix", "fp8"])
def test_native_abi_check(precision):
    assert os.path.exists(EXE), "tests/native/abi_check is not built (run __graft_entry__.build())"
    r = subprocess.run([EXE, precision], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "abi_check ok" in r.stdout, (r.returncode, r.stdout, r.stderr)

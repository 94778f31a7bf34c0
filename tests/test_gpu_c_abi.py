"""The C boundary from plain C (tests/c_abi/c_abi_check.c, built by
__graft_entry__.build()): device memory and a stream from the HIP runtime,
no Python between the caller and the library, every output against the fp64
C oracle (bar 2e-3, bf16 inputs, fp32 output); its first calls come from
four host threads at once."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "_build", "c_abi_check")


def test_c_program_against_the_oracle():
    if not os.path.exists(BINARY):
        raise AssertionError("%s is missing: run __graft_entry__.build() first" % BINARY)
    print("[gpu-case] c_abi_check", flush=True)
    r = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI CHECK OK" in r.stdout
    assert r.stdout.count("ok  :") == 8 and "FAIL" not in r.stdout

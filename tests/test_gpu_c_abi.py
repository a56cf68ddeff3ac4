"""The C ABI from a plain C program (tests/c_abi/c_abi_check.c, built by
__graft_entry__.build()): every compute entry point (prefill, prefill with
log-sum-exp, backward, decode, paged decode, rotary embedding, final cap) on
HIP-runtime buffers against the CPU oracle, and the documented error statuses,
with no Python in the process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "c_abi_check")


def test_c_program_against_the_oracle():
    print("[case] plain-C consumer of the C ABI", flush=True)
    sys.stdout.flush()
    assert os.path.exists(EXE), "tests/c_abi/c_abi_check is missing: run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "c_abi_check ok" in r.stdout

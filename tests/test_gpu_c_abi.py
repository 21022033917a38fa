"""librax used from a plain C program (tests/c_abi/single_key.c): no PyTorch in its process,
device memory through the HIP runtime, the calls through include/librax.h. The program checks
that DECODE and EXTEND over one stored key return its V row bit for bit, and that a NULL
argument is refused; it is built on the CPU by __graft_entry__.build() and run here as a child
process."""

import os
import subprocess

import pytest

from prefix_cached_paged_amd import build as B

from parity import say

pytestmark = pytest.mark.gpu


def test_plain_c_program_single_key():
    if not os.path.exists(B.C_ABI_BIN):
        pytest.fail("tests/c_abi/single_key is not built: run __graft_entry__.build()")
    say("plain-C program: single key through kv_store, decode and extend")
    r = subprocess.run([B.C_ABI_BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "c-abi ok"

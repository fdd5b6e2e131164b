"""GPU: the C ABI used from plain C.  tests/c_abi/abi_example.c allocates
with hipMalloc, calls dt_allreduce / dt_reduce_scatter / dt_all_gather /
dt_all_to_all / dt_bucket_allreduce / dt_barrier through include/dt.h only,
and compares every result bit for bit with the linked CPU oracle.  It runs as
a child process (built by __graft_entry__.build())."""
import os
import subprocess

import pytest

from gpu_util import note

pytestmark = pytest.mark.gpu

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_example")


def test_plain_c_program_matches_the_oracle():
    if not os.path.exists(BINARY):
        pytest.fail(f"{BINARY} is not built: run __graft_entry__.build() (or tests/c_abi/build.py)")
    note("plain C program over the C ABI")
    res = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-2000:] + res.stderr[-2000:]

"""The C ABI used from a program with no Python and no torch
(tests/c_abi/fused_from_c.cpp, built by __graft_entry__.build()): HIP memory
from hipMalloc, ce_workspace_init and ce_fwd_bwd_fused on the null stream,
then ce_shards_fwd_bwd_fused on the same logits in three separately
allocated shards, then ce_linear_cross_entropy (the chunked head) with the
library's own MFMA GEMM engine, each checked inside the program against the
oracle's C library.  Run here as a child process."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "fused_from_c")


def test_fused_call_from_c():
    assert os.path.exists(BIN), f"{BIN} is not built (run __graft_entry__.build())"
    say("[c abi] running tests/c_abi/fused_from_c")
    r = subprocess.run([BIN], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    say(r.stdout.strip())
    assert (r.returncode == 0 and "c abi ok:" in r.stdout and "c abi ok (3 shards)" in r.stdout
            and "c abi ok (linear, native)" in r.stdout), r.stdout

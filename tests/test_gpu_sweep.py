"""A seeded random sweep of the one-launch calls against the FP64 oracle.

Each case draws its dtype, vocabulary size (1 to 200000, log-uniform), rows,
memory layout (contiguous, padded rows, a misaligned first column, the
transposed (SQ, B) view), share of ignored rows (none to all), smoothing
convention and weight, reduction, upstream gradient and chunk split, then runs
ce_fwd_bwd_fused, or ce_shards_fwd_bwd_fused over 1 to 16 shards cut at random
columns, and compares loss, n and every gradient element with the oracle at
the stated bar.  The cases are fixed by their seeds, so a failure names a
reproducible case.
"""
import math

import numpy as np
import pytest
import torch

import vce_sweep_cases as cases
from gpu_util import say
from test_gpu_parity import check_fused
from test_gpu_shards_fused import check_shards

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(cases.N_FUSED))
def test_fused_sweep(seed):
    c = cases.fused_case(seed)
    say(f"[sweep fused] seed {seed}: {c['what']}")
    check_fused(c["x"], c["t"], c["alpha"], c["reduce"], g=c["g"], split_chunks=c["K"], what=c["what"],
                smoothing=c["smoothing"], diag=False)


@pytest.mark.parametrize("seed", range(cases.N_SHARDS))
def test_shards_sweep(seed):
    c = cases.shard_case(seed)
    say(f"[sweep shards] seed {seed}: {c['what']}")
    check_shards(c["x"], c["t"], c["bounds"], c["alpha"], c["reduce"], g=c["g"], smoothing=c["smoothing"],
                 separate=c["separate"], what=c["what"])

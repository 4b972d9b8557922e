"""A seeded random sweep of every entry point against the FP64 oracle.

Each case draws its dtype, vocabulary size (1 to 200000, log-uniform), rows,
memory layout (contiguous, padded rows, a misaligned first column, the
transposed (SQ, B) view), share of ignored rows (none to all), smoothing
convention and weight (from seed 20000 on: logits of sigma up to 20, weights up
to 1), reduction, upstream gradient and chunk split, then runs
ce_fwd_bwd_fused; ce_shards_fwd_bwd_fused over 1 to 16 shards cut at random
columns; ce_forward_ex + ce_backward_inplace_ex (and the FP32-lse form
ce_forward + ce_backward_inplace); the three-call shard flow; or the chunked
linear head (on the linear tests' grid-valued inputs; even seeds on the
native GEMM engine, odd ones on the library), and compares loss, n,
lse and every gradient element with the oracle at the stated bar.  The
separate backward fed the forward's lse_aux pair takes no allowance; fed the
FP32 lse alone it takes that hand-off's (lse_allowance), and fed FP32 shard
statistics the exchange format's rounding (stats_allowance).  The cases are
fixed by their seeds, so a failure names a reproducible case.
"""
import pytest

import vce_sweep_cases as cases
from gpu_util import check_shard_flow, check_split, say
from test_gpu_parity import check_fused
from test_gpu_shards_fused import check_shards

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", cases.seeds(cases.N_FUSED))
def test_fused_sweep(seed):
    c = cases.fused_case(seed)
    say(f"[sweep fused] seed {seed}: {c['what']}")
    check_fused(c["x"], c["t"], c["alpha"], c["reduce"], g=c["g"], split_chunks=c["K"], what=c["what"],
                smoothing=c["smoothing"], diag=False)


@pytest.mark.parametrize("seed", cases.seeds(cases.N_SHARDS))
def test_shards_sweep(seed):
    c = cases.shard_case(seed)
    say(f"[sweep shards] seed {seed}: {c['what']}")
    check_shards(c["x"], c["t"], c["bounds"], c["alpha"], c["reduce"], g=c["g"], smoothing=c["smoothing"],
                 separate=c["separate"], what=c["what"])


@pytest.mark.parametrize("seed", cases.seeds(cases.N_SPLIT))
def test_forward_backward_sweep(seed):
    c = cases.split_case(seed)
    say(f"[sweep fwd+bwd] seed {seed}: {c['what']}")
    check_split(c["x"], c["t"], c["alpha"], c["reduce"], g=c["g"], smoothing=c["smoothing"], what=c["what"])


@pytest.mark.parametrize("seed", cases.seeds(cases.N_SHARD_FLOW))
def test_shard_flow_sweep(seed):
    c = cases.shard_flow_case(seed)
    say(f"[sweep shard flow] seed {seed}: {c['what']}")
    check_shard_flow(c["x"], c["t"], c["bounds"], c["alpha"], c["reduce"], g=c["g"], smoothing=c["smoothing"],
                     what=c["what"])


@pytest.mark.parametrize("seed", range(cases.N_LINEAR))
def test_linear_sweep(seed):
    from test_gpu_linear import check_linear, grid_inputs
    c = cases.linear_case(seed)
    say(f"[sweep linear] seed {seed}: {c['what']}")
    h, w, t = grid_inputs(c["N"], c["D"], c["V"], c["dtype"], seed=c["seed"], ignore_frac=c["ignore_frac"])
    check_linear(h, w, t, c["alpha"], c["reduce"], g=c["g"], chunk_rows=c["chunk"], smoothing=c["smoothing"],
                 what=c["what"], want_dh=c["want_dh"], want_dw=c["want_dw"], h_pad=c["h_pad"],
                 gemm="native" if seed % 2 == 0 else "library")

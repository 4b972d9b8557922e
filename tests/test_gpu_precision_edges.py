"""Precision edges, checked against the FP64 oracle at the usual bar.

- Smoothing weights near 1: q_t and p_t are then both far below 1, and the
  target's gradient s (p_t - q_t), formed as (1 - q_t) - (1 - p_t), would
  cancel between two numbers near 1.  The fused calls must still meet the FP32
  bar there, unsplit, split and over shards.
- Logits of sigma 20, where lse is around 50: the lse that the forward and the
  shard flow hand to a separate backward must stay within the FP32 budget
  (lse_budget), so a conversion from base 2 that carries the FP32 log2(e)'s
  rounding (0.13 ulp at lse = 48) on top of its own rounding is caught.
- The base-2 sums round m log2(e) once and reuse that value, so the rounding
  cancels: a one-column shard's sum must come out as 1.
- FP32 rows of 65 to 128 columns under smoothing weights above 1/2, where
  q_o = a / V reaches 1/128 and a p_j close to it cancels in s (p_j - q_o):
  every such case of the stress generator's seeds 40000-70000 (the region
  where its FP32 path once missed the bar by up to 1.2e-7), fused and over
  shards, now on the FP64 whole-row path.
- The separate backward fed the forward's lse_aux pair: confident targets
  (p_t up to 1 - 1e-7) and smoothing near 1, where the FP32 lse alone cannot
  resolve s (p_t - q_t), at the stated bar with no allowance.
"""
import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
import vce_sweep_cases as cases
from gpu_util import assert_lse, assert_lse_pair, check_shard_flow, check_split, orc, say, to_device_view
from test_gpu_parity import check_fused
from test_gpu_shards_fused import check_shards

pytestmark = pytest.mark.gpu


def _logits(shape, dtype, sigma, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(dtype)


@pytest.mark.parametrize("alpha", [0.9996257424354553, 0.9940828680992126])
@pytest.mark.parametrize("V,K", [(7502, 0), (7502, 48), (235, 0)])
def test_fused_target_with_smoothing_near_one(alpha, V, K):
    x = _logits((2, 6, V), torch.float32, 0.5, seed=V + K)
    t = workloads.random_targets((2, 6), V, seed=V + K, ignore_frac=0.1)
    check_fused(x, t, float(np.float32(alpha)), "sum", split_chunks=K, what=f"a={alpha} V={V} K={K}")


@pytest.mark.parametrize("S", [1, 7])
def test_shard_target_with_smoothing_near_one(S):
    V = 235
    x = _logits((3, 7, V), torch.float32, 0.5, seed=90 + S)
    t = workloads.random_targets((3, 7), V, seed=90 + S, ignore_frac=0.1)
    check_shards(x, t, workloads.shard_bounds(V, S), float(np.float32(0.9955554604530334)), "none",
                 what=f"a near 1 S={S}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [27, 153, 1859, 22995])
def test_forward_lse_budget_at_sigma_20(dtype, V):
    x = _logits((4, 24, V), dtype, 20.0, seed=V)
    t = workloads.random_targets((4, 24), V, seed=V, ignore_frac=0.1)
    say(f"[precision] forward lse sigma 20 V={V} {dtype}")
    xd, td = to_device_view(x), to_device_view(t)
    _, lse, aux, _ = vce.ce_forward_ex(xd, td, 0.0, "none")
    torch.cuda.synchronize()
    _, ref_lse = orc().loss_rows(x, t, 0.0)
    kept = t.reshape(-1).numpy() != -100
    assert_lse(lse.cpu().numpy()[kept], ref_lse[kept], V, f"forward V={V}")
    assert_lse_pair(lse.cpu().numpy()[kept], aux.cpu().numpy()[kept, 0], ref_lse[kept], V, f"forward pair V={V}")


@pytest.mark.parametrize("S", [1, 5])
def test_shard_flow_lse_budget_at_sigma_20(S):
    V = 1859
    x = _logits((4, 24, V), torch.float32, 20.0, seed=S)
    t = workloads.random_targets((4, 24), V, seed=S, ignore_frac=0.1)
    N = t.numel()
    say(f"[precision] shard flow lse sigma 20 S={S}")
    td = to_device_view(t)
    bounds = workloads.shard_bounds(V, S)
    stats = torch.empty((S, N, 4), dtype=torch.float32, device="cuda")
    for s, (lo, hi) in enumerate(bounds):
        vce.ce_shard_partial_stats(x[..., lo:hi].contiguous().cuda(), td, lo, V, stats=stats[s])
    _, lse, _ = vce.ce_shard_combine(stats, td, V, 0.0, "none")
    torch.cuda.synchronize()
    _, ref_lse = orc().loss_rows(x, t, 0.0)
    kept = t.reshape(-1).numpy() != -100
    assert_lse(lse.cpu().numpy()[kept], ref_lse[kept], V, f"shard flow S={S}")


@pytest.mark.parametrize("width", [1, 200])
def test_single_column_shard_sums_are_one(width):
    """A shard whose only finite column is its maximum has the natural-units
    sum exp(x - M) = 1 exactly, or 0 where that column is the row's target
    (d leaves the target's term out).  Width 1 takes the FP64 path of short
    shard rows; width 200 (the other columns masked, -inf) the FP32 streaming
    path, whose base-2 sum is taken against M log2(e) rounded to FP32 and
    converted back by the same rounded value: if the compiler fuses that
    product unrounded into one side only, the rounding no longer cancels and
    the sum drifts by up to ulp(M log2 e) (about 1e-6 at M = 25)."""
    S = 6
    V = S * width
    N = 64
    gen = torch.Generator().manual_seed(61)
    vals = torch.randn((4, 16, S), generator=gen) * 20.0
    x = torch.full((4, 16, V), -float("inf"))
    cols = [s * width + (width // 2) for s in range(S)]  # the finite column of each shard
    for s in range(S):
        x[..., cols[s]] = vals[..., s]
    t = workloads.random_targets((4, 16), V, seed=61)
    tf = t.reshape(-1)
    for r in range(0, N, 5):  # some rows' target is a shard's finite column
        tf[r] = cols[(r // 5) % S]
    td = to_device_view(t)
    for s in range(S):
        lo = s * width
        st = torch.empty((N, 4), dtype=torch.float32, device="cuda")
        vce.ce_shard_partial_stats(x[..., lo:lo + width].contiguous().cuda(), td, lo, V, stats=st)
        torch.cuda.synchronize()
        got = st.cpu().numpy()
        assert np.array_equal(got[:, 0], vals[..., s].reshape(-1).numpy()), f"shard {s}: max"
        owner = tf.numpy() == cols[s]
        assert np.all(got[owner, 1] == 0.0), f"shard {s}: the target's own term must be left out"
        err = np.abs(got[~owner, 1].astype(np.float64) - 1.0)
        assert err.max() <= 2.0 ** -22, f"shard {s}: sum off 1 by {err.max():.3e}"


def test_shard_flow_lse_budget_narrow_shards_sigma_20():
    V = 23
    bounds = [(0, 1), (1, 5), (5, 6), (6, 8), (8, 12), (12, 14), (14, 17), (17, 23)]
    x = _logits((4, 24, V), torch.float32, 20.0, seed=23102)
    t = workloads.random_targets((4, 24), V, seed=23102, ignore_frac=0.1)
    N = t.numel()
    say("[precision] shard flow lse sigma 20, eight narrow shards")
    td = to_device_view(t)
    stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device="cuda")
    for s, (lo, hi) in enumerate(bounds):
        vce.ce_shard_partial_stats(x[..., lo:hi].contiguous().cuda(), td, lo, V, stats=stats[s])
    _, lse, _ = vce.ce_shard_combine(stats, td, V, 0.0, "none")
    torch.cuda.synchronize()
    _, ref_lse = orc().loss_rows(x, t, 0.0)
    kept = t.reshape(-1).numpy() != -100
    assert_lse(lse.cpu().numpy()[kept], ref_lse[kept], V, "shard flow, narrow shards")


def test_reading15_fused_wide_short_rows():
    """FP32 fused rows of 65-128 columns, smoothing above 1/2: every such
    case of stress seeds 40000-70000."""
    seeds = cases.wide_short_row_seeds("fused", 40000, 70000, 65, 128, 0.5)
    assert len(seeds) > 100
    for seed in seeds:
        c = cases.fused_case(seed)
        say(f"[reading 15 fused] seed {seed}: {c['what']}")
        check_fused(c["x"], c["t"], c["alpha"], c["reduce"], g=c["g"], split_chunks=c["K"], what=c["what"],
                    smoothing=c["smoothing"], diag=False)


def test_reading15_shards_wide_short_rows():
    """The same region over 1 to 16 shards (one launch)."""
    seeds = cases.wide_short_row_seeds("shards", 40000, 70000, 65, 128, 0.5)
    assert len(seeds) > 100
    for seed in seeds:
        c = cases.shard_case(seed)
        say(f"[reading 15 shards] seed {seed}: {c['what']}")
        check_shards(c["x"], c["t"], c["bounds"], c["alpha"], c["reduce"], g=c["g"], smoothing=c["smoothing"],
                     separate=c["separate"], what=c["what"])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [5000, 70001])
def test_split_calls_confident_targets(dtype, V):
    """p_t from about 0.6 to 1 - 1e-7: through lse_aux the target's gradient
    is s ((1 - q_t) - (1 - p_t)) with 1 - p_t from a sum without the target,
    as in the fused call, so no allowance is needed (the FP32 lse alone would
    resolve it to ulp(lse) only)."""
    g = torch.Generator().manual_seed(V)
    x = torch.randn((2, 8, V), generator=g)
    t = torch.randint(0, V, (2, 8), generator=g)
    for k in range(16):
        x.view(16, V)[k, t.view(-1)[k]] = 9.0 + 1.2 * k
    x = x.to(dtype)
    check_split(x, t, 0.0, False, what=f"confident V={V} {dtype}", legacy=False)
    check_split(x, t, 0.1, "mean", what=f"confident smoothed V={V} {dtype}", legacy=False)
    check_shard_flow(x, t, workloads.shard_bounds(V, 3), 0.1, "sum", what=f"confident shards V={V} {dtype}",
                     legacy=False, allowance=False)


@pytest.mark.parametrize("alpha", [0.9996257424354553, 0.9940828680992126])
@pytest.mark.parametrize("V", [7502, 235])
def test_split_calls_smoothing_near_one(alpha, V):
    x = _logits((2, 6, V), torch.float32, 0.5, seed=V + 1)
    t = workloads.random_targets((2, 6), V, seed=V + 1, ignore_frac=0.1)
    a = float(np.float32(alpha))
    check_split(x, t, a, "sum", what=f"split a={alpha} V={V}", legacy=False)
    check_shard_flow(x, t, workloads.shard_bounds(V, 4), a, "none", what=f"shard flow a={alpha} V={V}",
                     legacy=False, allowance=False)


@pytest.mark.parametrize("V", [2, 3, 5, 8, 40, 128])
def test_split_calls_few_columns_heavy_smoothing(V):
    """A vocabulary of a few columns under heavy smoothing puts p_j close to a
    large q_j: the forward + backward pair recomputes such rows in FP64, the
    shard flow's backward works in FP64 from the handed-over lse (within the
    FP32 statistics' rounding)."""
    x = _logits((4, 24, V), torch.float32, 1.0, seed=300 + V)
    t = workloads.random_targets((4, 24), V, seed=300 + V, ignore_frac=0.1)
    for a, sm in ((0.42, "all"), (0.9, "all"), (0.7, "others")):
        check_split(x, t, a, "none", g=np.linspace(-2.0, 2.0, 96), smoothing=sm, what=f"V={V} a={a} {sm}")
        if V >= 2:
            check_shard_flow(x, t, workloads.shard_bounds(V, min(V, 3)), a, "sum", g=1.7, smoothing=sm,
                             what=f"shards V={V} a={a} {sm}")

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
"""
import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import assert_lse, orc, say, to_device_view
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
    _, lse, _ = vce.ce_forward(xd, td, 0.0, "none")
    torch.cuda.synchronize()
    _, ref_lse = orc().loss_rows(x, t, 0.0)
    kept = t.reshape(-1).numpy() != -100
    assert_lse(lse.cpu().numpy()[kept], ref_lse[kept], V, f"forward V={V}")


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


def test_one_column_shard_sums_are_one():
    """A shard of one column holds only its maximum, so its natural-units sum
    exp(x - M) is exactly 1.  The base-2 sum is taken against M log2(e) rounded
    to FP32 and converted back by the same rounded value; if the compiler fuses
    that product unrounded into one side only, the rounding no longer cancels
    and the sum drifts by up to ulp(M log2 e) (about 1e-6 at M = 25)."""
    V = 6
    x = _logits((4, 16, V), torch.float32, 20.0, seed=61)
    t = workloads.random_targets((4, 16), V, seed=61)
    td = to_device_view(t)
    N = t.numel()
    for lo in range(V):
        st = torch.empty((N, 4), dtype=torch.float32, device="cuda")
        vce.ce_shard_partial_stats(x[..., lo:lo + 1].contiguous().cuda(), td, lo, V, stats=st)
        torch.cuda.synchronize()
        s = st.cpu().numpy()
        assert np.array_equal(s[:, 0], x[..., lo].reshape(-1).numpy()), f"column {lo}: max"
        err = np.abs(s[:, 1].astype(np.float64) - 1.0)
        assert err.max() <= 2.0 ** -22, f"column {lo}: sum off 1 by {err.max():.3e}"


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

"""Masked classes (logits of -inf) on the GPU against the FP64 oracle: the
loss leaves out zero-weight terms (0 log 0 = 0), so with no smoothing it
stays finite, with smoothing it is +inf, and a masked target makes it +inf;
gradients stay finite (the masked entries' gradient is -s q_o).  Two mask
patterns: the last columns (a vocabulary padded with masked entries) and
scattered columns, and one row whose target is masked.  Every entry point:
the fused call (the FP64 path of short rows, whole rows, split rows), forward
+ backward, and the shard flow.
"""
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import assert_grad, assert_grad_from_lse, assert_loss, orc, rows_f64, say, to_device_view

pytestmark = pytest.mark.gpu


def masked_case(dtype, V, pattern, seed, rows=(2, 9)):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((*rows, V), generator=g) * 2).to(dtype)
    t = workloads.random_targets(rows, V, seed=seed, ignore_frac=0.2)
    if pattern == "tail":
        pad = max(1, min(V // 8, 128))
        x[..., V - pad:] = -float("inf")
        masked = np.zeros(V, bool)
        masked[V - pad:] = True
    else:
        masked = np.zeros(V, bool)
        masked[torch.randperm(V, generator=g)[: max(1, V // 10)].numpy()] = True
        x[..., torch.as_tensor(masked)] = -float("inf")
    tf = t.reshape(-1)
    free = np.flatnonzero(~masked)
    for r in range(tf.numel()):  # keep targets off the mask, then mask one row's target
        if int(tf[r]) >= 0 and masked[int(tf[r])]:
            tf[r] = int(free[r % len(free)])
    r0 = int(np.flatnonzero(tf.numpy() >= 0)[0])
    tf[r0] = int(np.flatnonzero(masked)[0])
    return x, t


def assert_loss_inf(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isposinf(got), np.isposinf(ref)), f"{what}: inf rows differ: {got} vs {ref}"
    fin = np.isfinite(ref)
    assert not np.isnan(got).any(), f"{what}: NaN loss"
    assert_loss(got[fin], ref[fin], what)


CASES = [(dt, V, pat, K) for dt in (torch.bfloat16, torch.float32)
         for V, K in ((7, 0), (3001, 0), (8195, 3), (128000, 0)) for pat in ("tail", "scatter")]


@pytest.mark.parametrize("dtype,V,pattern,K", CASES,
                         ids=[f"{'bf16' if c[0] == torch.bfloat16 else 'f32'}-V{c[1]}-{c[2]}-K{c[3]}" for c in CASES])
@pytest.mark.parametrize("smoothing,alpha", [("all", 0.0), ("all", 0.1), ("others", 0.1)])
def test_fused_masked(dtype, V, pattern, K, smoothing, alpha):
    x, t = masked_case(dtype, V, pattern, seed=V + K)
    N = t.numel()
    o = orc()
    for reduce in ("none", "mean"):
        say(f"[masked fused] {dtype} V={V} {pattern} K={K} {smoothing} a={alpha} {reduce}")
        xd, td = to_device_view(x), to_device_view(t)
        g = np.linspace(0.5, 1.5, N) if reduce == "none" else 0.8
        gd = (torch.as_tensor(np.asarray(g, np.float32)).cuda() if reduce == "none"
              else torch.tensor([g], dtype=torch.float32, device="cuda"))
        loss, n = vce.ce_fwd_bwd_fused(xd, td, alpha, reduce, grad_out=gd, split_chunks=K, smoothing=smoothing)
        torch.cuda.synchronize()
        ref_rows, _ = o.loss_rows(x, t, alpha, smoothing=smoothing)
        if reduce == "none":
            assert_loss_inf(loss.cpu().numpy(), ref_rows, "masked loss rows")
        else:
            ref = o.reduce(ref_rows, reduce, o.count_valid(t))
            assert_loss_inf([loss.item()], [ref], "masked mean")
        grad = rows_f64(xd)
        assert np.all(np.isfinite(grad)), "masked: non-finite gradient"
        ref_g = o.grad_rows(x, t, alpha, reduce_loss=reduce, g=g, smoothing=smoothing)
        assert_grad(grad, ref_g, dtype, f"masked grad {reduce}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("alpha", [0.0, 0.1])
def test_forward_backward_masked(dtype, alpha):
    x, t = masked_case(dtype, 4099, "scatter", seed=77)
    N = t.numel()
    o = orc()
    ref_rows, ref_lse = o.loss_rows(x, t, alpha)
    ref_g = o.grad_rows(x, t, alpha, g=np.ones(N))
    kept = t.reshape(-1).numpy() != -100
    for form in ("ex", "lse"):
        say(f"[masked fwd+bwd {form}] {dtype} a={alpha}")
        xd, td = to_device_view(x), to_device_view(t)
        g = torch.ones(N, dtype=torch.float32, device="cuda")
        if form == "ex":
            loss, lse, aux, n = vce.ce_forward_ex(xd, td, alpha, False)
            vce.ce_backward_inplace_ex(xd, td, lse, aux, alpha, False, grad_out=g, n_valid=n)
        else:
            loss, lse, n = vce.ce_forward(xd, td, alpha, False)
            vce.ce_backward_inplace(xd, td, lse, alpha, False, grad_out=g, n_valid=n)
        torch.cuda.synchronize()
        assert_loss_inf(loss.cpu().numpy(), ref_rows, f"masked forward rows [{form}]")
        assert_loss(lse.cpu().numpy()[kept], ref_lse[kept], f"masked lse [{form}]")
        grad = rows_f64(xd)
        assert np.all(np.isfinite(grad))
        if form == "ex":
            assert_grad(grad, ref_g, dtype, "masked backward [ex]")
        else:
            # the FP32 lse alone: the rebuilt target gradient carries its resolution (as for unmasked rows)
            assert_grad_from_lse(grad, ref_g, dtype, lse.cpu().numpy(), t.reshape(-1).numpy(), np.ones(N),
                                 x.shape[-1], "masked backward [lse]")


@pytest.mark.parametrize("alpha", [0.0, 0.1])
def test_shard_flow_masked(alpha):
    V, S = 5003, 4
    x, t = masked_case(torch.bfloat16, V, "tail", seed=78)
    N = t.numel()
    bounds = workloads.shard_bounds(V, S)
    say(f"[masked shards] a={alpha}")
    td = to_device_view(t)
    shards = [x[..., a:b].contiguous().cuda() for a, b in bounds]
    stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device="cuda")
    for s, (a, b) in enumerate(bounds):
        vce.ce_shard_partial_stats(shards[s], td, a, V, stats=stats[s])
    loss, lse, aux, n = vce.ce_shard_combine_ex(stats, td, V, alpha, False)
    g = torch.ones(N, dtype=torch.float32, device="cuda")
    for s, (a, b) in enumerate(bounds):
        vce.ce_backward_inplace_ex(shards[s], td, lse, aux, alpha, False, grad_out=g, n_valid=n, vocab_start=a,
                                   vocab_total=V)
    torch.cuda.synchronize()
    o = orc()
    ref_rows, _ = o.loss_rows(x, t, alpha)
    assert_loss_inf(loss.cpu().numpy(), ref_rows, "masked shard loss")
    assert math.isfinite(float(lse.cpu().numpy()[t.reshape(-1).numpy() != -100].max()))
    ref_g = o.grad_rows(x, t, alpha, g=np.ones(N))
    for s, (a, b) in enumerate(bounds):
        grad = rows_f64(shards[s])
        assert np.all(np.isfinite(grad)), f"shard {s}: non-finite gradient"
        assert_grad(grad, ref_g[:, a:b], torch.bfloat16, f"masked shard {s}")

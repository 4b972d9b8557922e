"""A seeded random sweep of every entry point against the FP64 oracle.

Each case draws its dtype, vocabulary size (1 to 200000, log-uniform), rows,
memory layout (contiguous, padded rows, a misaligned first column, the
transposed (SQ, B) view), share of ignored rows (none to all), smoothing
convention and weight (from seed 20000 on: logits of sigma up to 20, weights up
to 1), reduction, upstream gradient and chunk split, then runs
ce_fwd_bwd_fused; ce_shards_fwd_bwd_fused over 1 to 16 shards cut at random
columns; ce_forward + ce_backward_inplace; the three-call shard flow; or the
chunked linear head (on the linear tests' grid-valued inputs), and
compares loss, n, lse and every gradient element with the oracle at the stated
bar (the calls that rebuild the gradient from an FP32 lse with that hand-off's
allowance at the target element).  The cases are fixed by their seeds, so a
failure names a reproducible case.
"""
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import vce_sweep_cases as cases
from gpu_util import (assert_grad_from_lse, assert_loss, assert_lse, ignored_rows, orc, raw_bits, rows_f64, say,
                      to_device_view)
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


def _g_dev(g, reduce, N):
    if reduce == "none":
        return torch.as_tensor(np.ones(N) if g is None else np.asarray(g), dtype=torch.float32).cuda()
    return torch.tensor([1.0 if g is None else float(g)], dtype=torch.float32, device="cuda")


def _scale(g, reduce, N, n):
    if reduce == "none":
        return np.ones(N) if g is None else np.asarray(g, np.float64)
    gg = 1.0 if g is None else float(g)
    return np.full(N, gg / n if reduce == "mean" else gg) if (reduce != "mean" or n) else np.full(N, np.nan)


def _softmax(x, t, lse_ref):
    """p_j = exp(x_j - lse) per logical row in FP64, for the lse hand-off's allowance; 0 on ignored rows,
    whose gradient must stay +0.0 exactly."""
    d0, d1, V = x.shape
    rows = x.reshape(d0 * d1, V).to(torch.float64).numpy()
    kept = t.reshape(-1).numpy() != -100
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(rows - np.asarray(lse_ref, np.float64)[:, None])
    p[~kept] = 0.0
    return p


def _check_loss(loss, ref_rows, reduce, n, o, what):
    if reduce == "none":
        assert_loss(loss.cpu().numpy().astype(np.float64), ref_rows, what + " rows")
    elif reduce == "mean" and n == 0:
        assert math.isnan(loss.item())
    else:
        assert_loss([loss.item()], [o.reduce(ref_rows, reduce, n)], f"{what} {reduce}")


@pytest.mark.parametrize("seed", cases.seeds(cases.N_SPLIT))
def test_forward_backward_sweep(seed):
    c = cases.split_case(seed)
    x, t, a, red, sm = c["x"], c["t"], c["alpha"], c["reduce"], c["smoothing"]
    N = t.numel()
    say(f"[sweep fwd+bwd] seed {seed}: {c['what']}")
    xd, td = to_device_view(x), to_device_view(t)
    loss, lse, n = vce.ce_forward(xd, td, a, red, smoothing=sm)
    vce.ce_backward_inplace(xd, td, lse, a, red, grad_out=_g_dev(c["g"], red, N), n_valid=n, smoothing=sm)
    torch.cuda.synchronize()
    o = orc()
    n_ref = o.count_valid(t)
    assert int(n.item()) == n_ref
    ref_rows, ref_lse = o.loss_rows(x, t, a, smoothing=sm)
    _check_loss(loss, ref_rows, red, n_ref, o, c["what"])
    kept = t.reshape(-1).numpy() != -100
    assert_lse(lse.cpu().numpy()[kept], ref_lse[kept], x.shape[-1], c["what"] + " lse")
    ref = o.grad_rows(x, t, a, reduce_loss=red, g=c["g"], n_valid=n_ref, smoothing=sm)
    tl = t.reshape(-1).numpy()
    assert_grad_from_lse(rows_f64(xd), ref, x.dtype, lse.cpu().numpy(), np.where(kept, tl, -1),
                         _scale(c["g"], red, N, n_ref), x.shape[-1], c["what"] + " grad", p=_softmax(x, t, ref_lse))
    ign = ignored_rows(t)
    assert not (len(ign) and raw_bits(xd, ign).any()), "ignored rows must be +0.0"


@pytest.mark.parametrize("seed", cases.seeds(cases.N_SHARD_FLOW))
def test_shard_flow_sweep(seed):
    c = cases.shard_flow_case(seed)
    x, t, a, red, sm, bounds = c["x"], c["t"], c["alpha"], c["reduce"], c["smoothing"], c["bounds"]
    N, V = t.numel(), c["V"]
    say(f"[sweep shard flow] seed {seed}: {c['what']}")
    td = to_device_view(t)
    shards = [x[..., lo:hi].contiguous().cuda() for lo, hi in bounds]
    stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device="cuda")
    for s, (lo, hi) in enumerate(bounds):
        vce.ce_shard_partial_stats(shards[s], td, lo, V, stats=stats[s])
    loss, lse, n = vce.ce_shard_combine(stats, td, V, a, red, smoothing=sm)
    for s, (lo, hi) in enumerate(bounds):
        vce.ce_backward_inplace(shards[s], td, lse, a, red, grad_out=_g_dev(c["g"], red, N), n_valid=n,
                                vocab_start=lo, vocab_total=V, smoothing=sm)
    torch.cuda.synchronize()
    o = orc()
    n_ref = o.count_valid(t)
    assert int(n.item()) == n_ref
    ref_rows, ref_lse = o.loss_rows(x, t, a, smoothing=sm)
    _check_loss(loss, ref_rows, red, n_ref, o, c["what"])
    kept = t.reshape(-1).numpy() != -100
    assert_lse(lse.cpu().numpy()[kept], ref_lse[kept], V, c["what"] + " lse")
    ref = o.grad_rows(x, t, a, reduce_loss=red, g=c["g"], n_valid=n_ref, smoothing=sm)
    tl = t.reshape(-1).numpy()
    sc = _scale(c["g"], red, N, n_ref)
    p = _softmax(x, t, ref_lse)
    for s, (lo, hi) in enumerate(bounds):
        local = np.where((tl >= lo) & (tl < hi), tl - lo, -1)
        assert_grad_from_lse(rows_f64(shards[s]), ref[:, lo:hi], x.dtype, lse.cpu().numpy(), local, sc, V,
                             f"{c['what']} shard {s}", p=p[:, lo:hi])
        ign = ignored_rows(t)
        assert not (len(ign) and raw_bits(shards[s], ign).any()), f"shard {s}: ignored rows must be +0.0"


@pytest.mark.parametrize("seed", range(cases.N_LINEAR))
def test_linear_sweep(seed):
    from test_gpu_linear import check_linear, grid_inputs
    c = cases.linear_case(seed)
    say(f"[sweep linear] seed {seed}: {c['what']}")
    h, w, t = grid_inputs(c["N"], c["D"], c["V"], c["dtype"], seed=c["seed"], ignore_frac=c["ignore_frac"])
    check_linear(h, w, t, c["alpha"], c["reduce"], g=c["g"], chunk_rows=c["chunk"], smoothing=c["smoothing"],
                 what=c["what"], want_dh=c["want_dh"], want_dw=c["want_dw"], h_pad=c["h_pad"])

"""Helpers for the GPU parity tests: move seeded host inputs to the device
with their exact layout, run the library, and compare with the FP64 oracle
under the parity bar:

  * n_valid, and the loss and gradient of ignored rows: bit-exact
    (ignored gradients are +0.0, bit pattern 0);
  * loss: |gpu - ref| <= 1e-4 * max(1, |ref|);
  * gradient: |gpu - ref| <= 2^-8 |ref| + 1e-7 (BF16) or 1e-5 |ref| + 1e-8
    (FP32), the GPU value widened exactly to FP64.
"""
from __future__ import annotations

import sys

import math

import numpy as np
import torch

import oracle
import vocab_cross_entropy_amd as vce

LOSS_RTOL = 1e-4
GRAD_TOL = {torch.bfloat16: (2.0 ** -8, 1e-7), torch.float32: (1e-5, 1e-8)}

_orc = None


def orc() -> oracle.Oracle:
    global _orc
    if _orc is None:
        _orc = oracle.default()
    return _orc


def say(msg: str):
    """Name the case on stdout before a GPU step (flushes)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_view(view: torch.Tensor, device="cuda") -> torch.Tensor:
    """Copy the whole storage of a CPU view to the device and rebuild the same
    view (shape, strides, storage offset) over it."""
    base = torch.empty(0, dtype=view.dtype).set_(view.untyped_storage())
    dev = base.to(device)
    return dev.as_strided(view.shape, view.stride(), view.storage_offset())


def rows_f64(x: torch.Tensor, rows=None) -> np.ndarray:
    """Logical rows of a (d0, d1, V) tensor as float64 (exact widening)."""
    d0, d1, V = x.shape
    flat = x.reshape(d0 * d1, V)
    if rows is not None:
        flat = flat[torch.as_tensor(rows, device=flat.device)]
    return flat.to(torch.float64).cpu().numpy()


def raw_bits(x: torch.Tensor, rows) -> np.ndarray:
    d0, d1, V = x.shape
    flat = x.reshape(d0 * d1, V)[torch.as_tensor(rows, device=x.device)]
    it = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
    return flat.contiguous().view(it).cpu().numpy()


def assert_loss(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    tol = LOSS_RTOL * np.maximum(1.0, np.abs(ref))
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: loss off at {np.flatnonzero(bad)[:5]} max err {np.nanmax(err):.3e}"


def assert_grad(gpu, ref, dtype, what="", floor_scale=1.0, extra_rtol=0.0, allow=None):
    """Elementwise gradient bar; ``floor_scale`` < 1 tightens the absolute
    floor (diagnostic check of g/s against ref/s), ``extra_rtol`` widens the
    relative term of that diagnostic; ``allow`` (an array like ref) adds a
    stated per-element slack."""
    rtol, atol = GRAD_TOL[dtype]
    err = np.abs(gpu - ref)
    tol = (rtol + extra_rtol) * np.abs(ref) + atol * floor_scale
    if allow is not None:
        tol = tol + allow
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: grad off at {len(np.argwhere(bad))} elements, first {tuple(i)} "
                             f"gpu {gpu[tuple(i)]!r} ref {ref[tuple(i)]!r} (max err {err.max():.3e})")


def ignored_rows(t: torch.Tensor, ignore_idx=-100) -> np.ndarray:
    return np.flatnonzero(t.reshape(-1).cpu().numpy() == ignore_idx)


def lse_budget(lse: np.ndarray, vocab: int) -> np.ndarray:
    """Budget for the error of an FP32 lse = m + log(d) over `vocab` columns,
    per row: ulp(lse) for rounding m + log(d), plus the relative error of the
    FP32 sum d = sum_j exp(x_j - m), which moves lse by as much.  Each term's
    exponential rounds by up to 2 units of 2^-24, and each addition that forms
    d by up to one unit of the partial sum.  The kernels give a row at least
    256 lanes, each summing whole 16-byte vectors (at most 8 columns) in
    sequence, chains of at most l = ceil(vocab / 256) + 10 additions, and then
    add the lanes in a tree of at most ceil(log2 vocab) levels.  A chain's
    roundings have random signs and grow like sqrt(l); the tree's levels, one
    unit each:
        budget = ulp(lse) + (2 + ceil(log2 vocab) + ceil(sqrt(l))) 2^-24.
    Near lse = 0 the sum's term dominates: at |lse| = 0.3 two roundings of a
    three-term d already come to 3.5 ulp(lse).  This is a realistic budget for
    that schedule, not a worst-case bound (a chain's worst case is l units)."""
    lse = np.abs(np.asarray(lse, dtype=np.float64))
    ulp = np.exp2(np.floor(np.log2(np.maximum(lse, 2.0 ** -126))) - 23)
    v = max(int(vocab), 1)
    chain = -(-v // 256) + 10
    return ulp + (2 + math.ceil(math.log2(v)) + math.ceil(math.sqrt(chain))) * 2.0 ** -24


def assert_lse(gpu, ref, vocab, what=""):
    """An FP32 lse that a separate backward will rebuild p_j from, within lse_budget of the FP64 value."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = ~(err <= lse_budget(ref, vocab))
    assert not bad.any(), (f"{what}: lse off at {np.flatnonzero(bad)[:5]}, first gpu {gpu[bad][0]!r} "
                           f"ref {ref[bad][0]!r}")


def lse_allowance(ref: np.ndarray, lse: np.ndarray, targets_local: np.ndarray, scale: np.ndarray,
                  vocab: int, p: np.ndarray | None = None) -> np.ndarray:
    """Extra absolute slack for gradients rebuilt from an FP32 lse
    (ce_backward_inplace): an error e in the lse it is handed scales every
    p_j = exp(x_j - lse) by about 1 - e.  Where p_t is close to 1 that is the
    whole of s (p_t - 1) at the target; where p_j sits close to a large q_j (a
    few columns, heavy smoothing) it is the whole of s (p_j - q_j).  The slack
    is |s| max(p_j, [j = t]) lse_budget(lse, vocab); with no p given, at the
    target element only.  The fused calls need none of it.
    targets_local[i] < 0: not in this buffer."""
    allow = np.zeros_like(ref)
    unit = np.abs(np.asarray(scale, dtype=np.float64)) * lse_budget(lse, vocab)
    if p is not None:
        allow = np.nan_to_num(np.asarray(p, dtype=np.float64) * unit[:, None])
    for i, j in enumerate(np.asarray(targets_local)):
        if 0 <= j < ref.shape[1]:
            allow[i, j] = max(allow[i, j], unit[i])
    return allow


def assert_grad_from_lse(gpu, ref, dtype, lse, targets_local, scale, vocab, what="", p=None):
    rtol, atol = GRAD_TOL[dtype]
    err = np.abs(gpu - ref)
    tol = rtol * np.abs(ref) + atol + lse_allowance(ref, lse, targets_local, scale, vocab, p)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: grad off at {len(np.argwhere(bad))} elements, first {tuple(i)} "
                             f"gpu {gpu[tuple(i)]!r} ref {ref[tuple(i)]!r} (max err {err.max():.3e})")


def sum_budget(vocab: int) -> float:
    """The part of lse_budget that the FP32 sum d contributes (no final rounding of lse)."""
    v = max(int(vocab), 1)
    chain = -(-v // 256) + 10
    return (2 + math.ceil(math.log2(v)) + math.ceil(math.sqrt(chain))) * 2.0 ** -24


def assert_lse_pair(hi, lo, ref, vocab, what=""):
    """lse + its handed-over residual: the FP32 sum's error only, without lse's own rounding."""
    got = np.asarray(hi, np.float64) + np.asarray(lo, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= sum_budget(vocab) + 2.0 ** -40 * np.abs(ref))
    assert not bad.any(), (f"{what}: lse pair off at {np.flatnonzero(bad)[:5]}, first {got[bad][0]!r} "
                           f"ref {ref[bad][0]!r}")


def stats_allowance(p: np.ndarray, targets_local: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Slack for a backward fed by FP32 shard statistics (the three-call shard
    flow): each exchanged d is one FP32 number, so the combined D and with it
    every p_j = exp(x_j - lse) carry at least its rounding, 2^-24 relative;
    1 - p_t = D_excl / D twice that.  Where p_j sits close to a large q_j (a
    vocabulary of a few columns under heavy smoothing) that rounding is the
    whole of s (p_j - q_j).  Allowed: |s| max(p_j, [j = t]) 2^-22 (a factor two
    over the rounding's bound).  targets_local[i] < 0: not in this buffer."""
    unit = np.abs(np.asarray(scale, np.float64)) * 2.0 ** -22
    allow = np.nan_to_num(np.asarray(p, np.float64) * unit[:, None])
    for i, j in enumerate(np.asarray(targets_local)):
        if 0 <= j < allow.shape[1]:
            allow[i, j] = max(allow[i, j], unit[i])
    return allow


def reduced(reduce) -> bool:
    """True for the mean (True / "mean") and the sum ("sum")."""
    return oracle.reduction_code(reduce) != 0


def g_device(g, reduce, N):
    """The upstream gradient on the device: None (1), a scalar (mean, sum) or [N] values."""
    if g is None:
        return None
    if reduced(reduce):
        return torch.tensor([float(g)], dtype=torch.float32, device="cuda")
    return torch.as_tensor(np.asarray(g, dtype=np.float32).reshape(N), device="cuda")


def row_scales(g, reduce, N, n):
    """s_i of every row: g_i (none), g / n (mean; NaN with n = 0), g (sum)."""
    code = oracle.reduction_code(reduce)
    if code == 0:
        return np.ones(N) if g is None else np.asarray(g, np.float64).reshape(N)
    gg = 1.0 if g is None else float(g)
    if code == 1:
        return np.full(N, gg / n) if n else np.full(N, np.nan)
    return np.full(N, gg)


def softmax_rows(x, t, lse_ref, ignore_idx=-100):
    """p_j = exp(x_j - lse) per logical row in FP64 from the oracle's lse, for
    the allowances above; 0 on ignored rows, whose gradient must stay +0.0."""
    d0, d1, V = x.shape
    rows = x.reshape(d0 * d1, V).to(torch.float64).numpy()
    kept = t.reshape(-1).numpy() != ignore_idx
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(rows - np.asarray(lse_ref, np.float64)[:, None])
    p[~kept] = 0.0
    return p


def _check_reduced_loss(loss, ref_rows, reduce, n, what):
    o = orc()
    if not reduced(reduce):
        assert_loss(loss.cpu().numpy().astype(np.float64), ref_rows, what + " rows")
    elif oracle.reduction_code(reduce) == 1 and n == 0:
        assert math.isnan(loss.item()), f"{what}: mean of no rows must be NaN"
    else:
        assert_loss([loss.item()], [o.reduce(ref_rows, reduce, n)], f"{what} {reduce}")


def check_split(x, t, alpha, reduce, g=None, smoothing="all", what="", legacy=True, masked=False):
    """ce_forward_ex + ce_backward_inplace_ex on a device copy of (x, t),
    compared with the oracle at the stated bar, with no allowance; with
    ``legacy``, ce_forward + ce_backward_inplace (the FP32 lse alone) on another
    copy, at the bar plus lse_allowance, the resolution of that hand-off.
    ``masked``: logits hold -inf, lse is then not compared (it may be -inf)."""
    d0, d1, V = x.shape
    N = d0 * d1
    o = orc()
    n_ref = o.count_valid(t)
    ref_rows, ref_lse = o.loss_rows(x, t, alpha, smoothing=smoothing)
    ref = o.grad_rows(x, t, alpha, reduce_loss=reduce, g=g, n_valid=n_ref, smoothing=smoothing)
    kept = t.reshape(-1).numpy() != -100
    tl = np.where(kept, t.reshape(-1).numpy(), -1)
    ign = ignored_rows(t)
    for form in ("ex", "lse") if legacy else ("ex",):
        say(f"[split {form}] {what} shape={tuple(x.shape)} {x.dtype} a={alpha} {reduce} {smoothing}")
        xd, td = to_device_view(x), to_device_view(t)
        gd = g_device(g, reduce, N)
        if form == "ex":
            loss, lse, aux, n = vce.ce_forward_ex(xd, td, alpha, reduce, smoothing=smoothing)
            vce.ce_backward_inplace_ex(xd, td, lse, aux, alpha, reduce, grad_out=gd, n_valid=n, smoothing=smoothing)
        else:
            loss, lse, n = vce.ce_forward(xd, td, alpha, reduce, smoothing=smoothing)
            vce.ce_backward_inplace(xd, td, lse, alpha, reduce, grad_out=gd, n_valid=n, smoothing=smoothing)
        torch.cuda.synchronize()
        assert int(n.item()) == n_ref, f"{what}: n {int(n.item())} != {n_ref}"
        _check_reduced_loss(loss, ref_rows, reduce, n_ref, f"{what} [{form}]")
        lv = lse.cpu().numpy()
        assert not lv[~kept].view(np.int32).any(), f"{what}: ignored rows' lse must be +0.0"
        if not masked:
            assert_lse(lv[kept], ref_lse[kept], V, f"{what} [{form}] lse")
            if form == "ex":
                av = aux.cpu().numpy()
                assert_lse_pair(lv[kept], av[kept, 0], ref_lse[kept], V, f"{what} lse pair")
        gpu = rows_f64(xd)
        if form == "ex":
            assert_grad(gpu, ref, x.dtype, f"{what} [ex] grad")
        else:
            assert_grad_from_lse(gpu, ref, x.dtype, lv, tl, row_scales(g, reduce, N, n_ref), V,
                                 f"{what} [lse] grad", p=softmax_rows(x, t, ref_lse))
        assert not (len(ign) and raw_bits(xd, ign).any()), f"{what} [{form}]: ignored rows must be +0.0"


def check_shard_flow(x, t, bounds, alpha, reduce, g=None, smoothing="all", what="", legacy=True, masked=False,
                     allowance=True):
    """The three-call shard flow on contiguous copies of x's column ranges
    ``bounds``: ce_shard_partial_stats per shard, ce_shard_combine_ex, then
    ce_backward_inplace_ex per shard from the combine's lse and lse_aux,
    compared with the oracle at the stated bar plus stats_allowance (the FP32
    exchanged statistics; none with ``allowance=False``); with ``legacy``, the
    same flow handing over the FP32 lse alone, at the bar plus lse_allowance.
    Returns the ex flow's statistics [S, N, 4] and loss."""
    d0, d1, V = x.shape
    N = d0 * d1
    o = orc()
    n_ref = o.count_valid(t)
    ref_rows, ref_lse = o.loss_rows(x, t, alpha, smoothing=smoothing)
    ref = o.grad_rows(x, t, alpha, reduce_loss=reduce, g=g, n_valid=n_ref, smoothing=smoothing)
    kept = t.reshape(-1).numpy() != -100
    tl = np.where(kept, t.reshape(-1).numpy(), -1)
    sc = row_scales(g, reduce, N, n_ref)
    p = softmax_rows(x, t, ref_lse)
    ign = ignored_rows(t)
    out = None
    for form in ("ex", "lse") if legacy else ("ex",):
        say(f"[shard flow {form}] {what} S={len(bounds)} {x.dtype} a={alpha} {reduce} {smoothing}")
        td = to_device_view(t)
        shards = [x[..., lo:hi].contiguous().cuda() for lo, hi in bounds]
        stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device="cuda")
        for s, (lo, hi) in enumerate(bounds):
            vce.ce_shard_partial_stats(shards[s], td, lo, V, stats=stats[s])
        gd = g_device(g, reduce, N)
        if form == "ex":
            loss, lse, aux, n = vce.ce_shard_combine_ex(stats, td, V, alpha, reduce, smoothing=smoothing)
        else:
            loss, lse, n = vce.ce_shard_combine(stats, td, V, alpha, reduce, smoothing=smoothing)
            aux = None
        for s, (lo, hi) in enumerate(bounds):
            vce.ce_backward_inplace_ex(shards[s], td, lse, aux, alpha, reduce, grad_out=gd, n_valid=n,
                                       vocab_start=lo, vocab_total=V, smoothing=smoothing)
        torch.cuda.synchronize()
        assert int(n.item()) == n_ref, f"{what}: n {int(n.item())} != {n_ref}"
        _check_reduced_loss(loss, ref_rows, reduce, n_ref, f"{what} [{form}]")
        lv = lse.cpu().numpy()
        if not masked:
            assert_lse(lv[kept], ref_lse[kept], V, f"{what} [{form}] lse")
        for s, (lo, hi) in enumerate(bounds):
            local = np.where((tl >= lo) & (tl < hi), tl - lo, -1)
            gpu = rows_f64(shards[s])
            if form == "ex":
                assert_grad(gpu, ref[:, lo:hi], x.dtype, f"{what} [ex] shard {s}",
                            allow=stats_allowance(p[:, lo:hi], local, sc) if allowance else None)
            else:
                assert_grad_from_lse(gpu, ref[:, lo:hi], x.dtype, lv, local, sc, V, f"{what} [lse] shard {s}",
                                     p=p[:, lo:hi])
            assert not (len(ign) and raw_bits(shards[s], ign).any()), f"{what} shard {s}: ignored rows not +0.0"
        if form == "ex":
            out = (stats, loss)
    return out

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


def assert_grad(gpu, ref, dtype, what="", floor_scale=1.0, extra_rtol=0.0):
    """Elementwise gradient bar; ``floor_scale`` < 1 tightens the absolute
    floor (diagnostic check of g/s against ref/s), ``extra_rtol`` widens the
    relative term of that diagnostic."""
    rtol, atol = GRAD_TOL[dtype]
    err = np.abs(gpu - ref)
    tol = (rtol + extra_rtol) * np.abs(ref) + atol * floor_scale
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

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


def lse_allowance(ref: np.ndarray, lse: np.ndarray, targets_local: np.ndarray, scale: np.ndarray,
                  p: np.ndarray | None = None) -> np.ndarray:
    """Extra absolute slack for gradients rebuilt from an FP32 lse
    (ce_backward_inplace): the hand-off rounds lse by up to half an ulp, which
    scales every p_j = exp(x_j - lse) by about that much.  Where p_t is close
    to 1 that is the whole of s (p_t - 1) at the target; where p_j sits close
    to a large q_j (a few columns, heavy smoothing) it is the whole of
    s (p_j - q_j).  The slack is |s| max(p_j, [j = t]) (ulp(lse) + 2^-24); with
    no p given, at the target element only.  The fused calls need none of it.
    targets_local[i] < 0: not in this buffer."""
    allow = np.zeros_like(ref)
    lse = np.abs(np.asarray(lse, dtype=np.float64))
    ulp = np.exp2(np.floor(np.log2(np.maximum(lse, 2.0 ** -126))) - 23)
    unit = np.abs(np.asarray(scale, dtype=np.float64)) * (ulp + 2.0 ** -24)
    if p is not None:
        allow = np.nan_to_num(np.asarray(p, dtype=np.float64) * unit[:, None])
    for i, j in enumerate(np.asarray(targets_local)):
        if 0 <= j < ref.shape[1]:
            allow[i, j] = max(allow[i, j], unit[i])
    return allow


def assert_grad_from_lse(gpu, ref, dtype, lse, targets_local, scale, what="", p=None):
    rtol, atol = GRAD_TOL[dtype]
    err = np.abs(gpu - ref)
    tol = rtol * np.abs(ref) + atol + lse_allowance(ref, lse, targets_local, scale, p)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: grad off at {len(np.argwhere(bad))} elements, first {tuple(i)} "
                             f"gpu {gpu[tuple(i)]!r} ref {ref[tuple(i)]!r} (max err {err.max():.3e})")

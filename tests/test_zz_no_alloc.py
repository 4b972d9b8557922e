"""The allocation-free fused call, ce_fwd_bwd_fused_noalloc, through the C ABI.

Its workspace is the library's static per-device array, so the call takes no
workspace and allocates nothing.  Checked against ce_fwd_bwd_fused (same
kernels, a caller-provided workspace) on the same inputs, bit for bit, and
against the FP64 oracle, on two calls in a row, the second with a smaller
input (the array keeps the first call's words; the tagged-word protocol must
not take them for the second call's), and with the device's free memory the
same before and after.
"""
import ctypes

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import assert_loss, orc, say, to_device_view
from vocab_cross_entropy_amd import _abi

pytestmark = pytest.mark.gpu


def _case(shape, V, dtype, seed, ignore_frac=0.05):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((*shape, V), generator=g) * 2).to(dtype)
    t = workloads.random_targets(shape, V, seed=seed, ignore_frac=ignore_frac)
    return x, t


def _noalloc(xd, td, alpha, reduce, grad_out, loss, n_valid, split_chunks=0, smoothing="all"):
    """One call of the entry point itself through ctypes (no binding logic)."""
    p = vce.params(alpha, reduce, -100, split_chunks, smoothing)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = vce.lib.ce_fwd_bwd_fused_noalloc(ctypes.byref(vce.logits_desc(xd)), ctypes.byref(vce.targets_desc(td)),
                                          ctypes.byref(p), None if grad_out is None else grad_out.data_ptr(),
                                          loss.data_ptr(), n_valid.data_ptr(), stream)
    assert rc == _abi.CE_OK, vce.lib.ce_last_error().decode()


def _check_pair(x, t, alpha, reduce, g, split_chunks, what, outs):
    """The reference call on one copy, then the allocation-free call on
    another into the preallocated ``outs`` = (loss, n_valid); both compared."""
    N = t.numel()
    say(f"[noalloc] {what}: reference ce_fwd_bwd_fused")
    td = to_device_view(t)
    xa = to_device_view(x)
    gd = None if g is None else (torch.tensor([g], dtype=torch.float32, device="cuda") if reduce != "none"
                                 else torch.as_tensor(np.asarray(g, np.float32), device="cuda"))
    loss_a, n_a = vce.ce_fwd_bwd_fused(xa, td, alpha, reduce, grad_out=gd, split_chunks=split_chunks)
    xb = to_device_view(x)
    loss_b, n_b = outs
    loss_b.fill_(float("nan"))
    n_b.fill_(-7)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    say(f"[noalloc] {what}: ce_fwd_bwd_fused_noalloc")
    _noalloc(xb, td, alpha, reduce, gd, loss_b, n_b, split_chunks)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "device memory changed across the allocation-free call"
    nl = 1 if reduce != "none" else N
    assert int(n_b.item()) == int(n_a.item()) == orc().count_valid(t)
    assert torch.equal(loss_b[:nl].view(torch.int32), loss_a.view(torch.int32)), f"{what}: loss differs"
    view = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(xb.view(view), xa.view(view)), f"{what}: gradient differs"
    ref_rows, _ = orc().loss_rows(x, t, alpha)
    if reduce == "none":
        assert_loss(loss_b[:nl].cpu().numpy().astype(np.float64), ref_rows, what)
    else:
        assert_loss([loss_b[0].item()], [orc().reduce(ref_rows, reduce, orc().count_valid(t))], what)


def test_two_calls_in_a_row_second_smaller():
    # outputs preallocated once, for the larger call
    loss = torch.empty(2 * 40, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    # 1: rows split over 4 workgroups (the 128000-column BF16 shape), mean
    x, t = _case((2, 40), 128000, torch.bfloat16, seed=701)
    _check_pair(x, t, 0.1, "mean", None, 0, "128000 columns, mean", (loss, n))
    # 2: fewer, shorter rows, forced into 3 chunks, per-row upstream gradient
    x, t = _case((3, 5), 12003, torch.bfloat16, seed=702, ignore_frac=0.2)
    _check_pair(x, t, 0.0, "none", np.linspace(-1.0, 2.0, 15), 3, "12003 columns, K = 3, none", (loss, n))
    # 3: still smaller: FP32 rows of 100 columns (the FP64 whole-row path), sum
    x, t = _case((2, 3), 100, torch.float32, seed=703)
    _check_pair(x, t, 0.6, "sum", 0.5, 0, "100 columns FP32, sum", (loss, n))

"""The autograd form (parallel_cross_entropy / ParallelCrossEntropy) on the
GPU, through the C ABI, against the FP64 oracle, and its memory behaviour
(TENPU #29 section 6: peak within 5% of PyTorch's cross-entropy, no growth
over repeated calls).

The forward stages the gradient for an upstream gradient of 1 in place; the
backward multiplies it by the upstream gradient (ce_scale_grad_inplace).  For
a factor that is 1 or a power of two the result is exactly what a direct call
with that factor gives, so the stated bar applies.  For any other factor a
BF16 gradient is rounded twice (once staged, once scaled), each rounding
within half a BF16 ulp, so those cases allow 2 x 2^-8 |ref|; FP32 keeps its bar.
"""
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import GRAD_TOL, assert_grad, assert_loss, ignored_rows, orc, raw_bits, rows_f64, say, to_device_view

pytestmark = pytest.mark.gpu


def _inputs(dtype, shape=(2, 9), V=4099, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(*shape, V, generator=g) * 2).to(dtype)
    t = workloads.random_targets(shape, V, seed=seed, ignore_frac=0.25)
    return x, t


CASES = [(dt, red, gk) for dt in (torch.bfloat16, torch.float32) for red in (False, True)
         for gk in ("one", "pow2", "any", "neg")]


@pytest.mark.parametrize("dtype,reduce,gkind", CASES,
                         ids=[f"{'bf16' if c[0] == torch.bfloat16 else 'f32'}-{'mean' if c[1] else 'rows'}-{c[2]}"
                              for c in CASES])
def test_backward_matches_oracle(dtype, reduce, gkind):
    x, t = _inputs(dtype, seed=3 + CASES.index((dtype, reduce, gkind)))
    N = t.numel()
    o = orc()
    n = o.count_valid(t)
    rng = np.random.default_rng(5)
    if reduce:
        gval = {"one": 1.0, "pow2": 0.25, "any": 0.3, "neg": -1.7}[gkind]
        g_host = np.float32(gval)
        grad_arg = torch.tensor(gval, dtype=torch.float32, device="cuda")
        g_or = float(g_host)
    else:
        g_host = {"one": np.ones(N), "pow2": np.full(N, 0.5), "any": rng.uniform(0.1, 3.0, N),
                  "neg": -rng.uniform(0.1, 3.0, N)}[gkind].astype(np.float32)
        g_host[0] = 1.0  # a row left untouched by the scale
        grad_arg = torch.as_tensor(g_host, device="cuda").view(t.shape)
        g_or = g_host.astype(np.float64)
    say(f"[autograd] {dtype} reduce={reduce} g={gkind}")
    xd = to_device_view(x).requires_grad_(True)
    td = to_device_view(t)
    loss = vce.parallel_cross_entropy(xd, td, label_smoothing=0.1, reduce_loss=reduce)
    loss.backward(grad_arg)
    torch.cuda.synchronize()
    ref_rows, _ = o.loss_rows(x, t, 0.1)
    if reduce:
        assert_loss([float(loss.item())], [o.mean_loss(ref_rows, n)], "autograd mean loss")
    else:
        assert_loss(loss.detach().reshape(-1).cpu().numpy(), ref_rows, "autograd row loss")
    assert xd.grad is not None and xd.grad.data_ptr() == xd.data_ptr()  # the gradient lives in inp's storage
    ref = o.grad_rows(x, t, 0.1, reduce_loss=reduce, g=g_or, n_valid=n)
    got = rows_f64(xd.grad)
    exact_factor = gkind in ("one", "pow2") or dtype == torch.float32
    if exact_factor:
        assert_grad(got, ref, dtype, "autograd grad")
    else:
        rtol, atol = GRAD_TOL[dtype]
        gmax = float(np.max(np.abs(g_or)))
        err = np.abs(got - ref)
        bad = ~(err <= 2 * rtol * np.abs(ref) + atol * max(1.0, gmax))
        assert not bad.any(), f"autograd grad (two roundings): {bad.sum()} elements, max err {err.max():.3e}"
    ign = ignored_rows(t)
    if len(ign):
        assert not raw_bits(xd.grad.detach(), ign).any(), "ignored rows must stay +0.0 for any upstream gradient"


def test_backward_through_a_matmul():
    """Logits produced by a matmul: the staged gradient flows into the
    weights' gradient (W.grad = h^T dL/dlogits)."""
    g = torch.Generator().manual_seed(17)
    Nr, Dm, V = 48, 64, 3000
    h = (torch.randn(Nr, Dm, generator=g) * 0.5).cuda()
    W = (torch.randn(Dm, V, generator=g) * 0.5).cuda().requires_grad_(True)
    t = workloads.random_targets((2, Nr // 2), V, seed=17, ignore_frac=0.1)
    td = t.cuda()
    logits = (h @ W).view(2, Nr // 2, V)
    logits_host = logits.detach().cpu().clone()  # the values the kernel will read
    loss = vce.parallel_cross_entropy(logits, td, label_smoothing=0.0, reduce_loss=True)
    loss.backward()
    torch.cuda.synchronize()
    o = orc()
    grad_logits = o.grad_rows(logits_host, t, 0.0, reduce_loss=True, n_valid=o.count_valid(t))
    ref = h.double().cpu().numpy().T @ grad_logits
    got = W.grad.double().cpu().numpy()
    err = np.abs(got - ref)
    assert np.all(err <= 1e-4 * np.abs(ref) + 1e-7), f"W.grad off: max err {err.max():.3e}"


def test_memory_peak_within_five_percent():
    """Peak device memory of forward + backward over what the inputs hold:
    at most 5% of the logits' size (the pages' target is 5% over PyTorch's
    cross-entropy, which needs whole N x V intermediates and a gradient)."""
    x, t = _inputs(torch.bfloat16, shape=(4, 1024), V=32000, seed=21)
    xd, td = to_device_view(x).requires_grad_(True), to_device_view(t)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    loss = vce.parallel_cross_entropy(xd, td, label_smoothing=0.1, reduce_loss=True)
    loss.backward()
    torch.cuda.synchronize()
    ours = torch.cuda.max_memory_allocated() - base
    # PyTorch's cross-entropy on a fresh copy, for the comparison the pages make
    xr = to_device_view(x).requires_grad_(True)
    torch.cuda.synchronize()
    base_t = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    lt = torch.nn.functional.cross_entropy(xr.view(-1, xr.shape[-1]), td.view(-1), ignore_index=-100,
                                           label_smoothing=0.1)
    lt.backward()
    torch.cuda.synchronize()
    theirs = torch.cuda.max_memory_allocated() - base_t
    say(f"[memory] peak over inputs: ours {ours} B, torch {theirs} B, logits {xd.numel() * xd.element_size()} B")
    assert ours <= 0.05 * xd.numel() * xd.element_size()
    assert ours <= 1.05 * theirs


def test_memory_no_growth_over_repeated_calls():
    x, t = _inputs(torch.bfloat16, shape=(2, 64), V=8192, seed=23)
    xd, td = to_device_view(x).requires_grad_(True), to_device_view(t)
    pristine = xd.detach().clone()
    torch.cuda.synchronize()
    before = None
    for i in range(30):
        with torch.no_grad():
            xd.copy_(pristine)
        xd.grad = None
        loss = vce.parallel_cross_entropy(xd, td, label_smoothing=0.1, reduce_loss=True)
        loss.backward()
        del loss
        torch.cuda.synchronize()
        if i == 2:
            before = torch.cuda.memory_allocated()
    assert torch.cuda.memory_allocated() == before

"""The option flags on the GPU, through the C ABI, against the FP64 oracle:

  * smoothing over the V - 1 classes other than the target (the CANN ops-nn
    page's kernel: forward step 4, backward "pitfall 3"), next to torch's
    a / V over all classes;
  * the sum reduction, and the sum over an external count of valid tokens
    (hyper-parallel issue #269, comparison table row "reduction semantics":
    Titan's training default), passed as the upstream gradient 1 / count.

Every entry point that uses the smoothing or the reduction is covered: the
fused call (whole and split rows, the register-reuse path of BF16), forward
+ backward, the vocabulary-shard flow and the autograd form.  Same bar as the
other parity tests (gpu_util).
"""
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import (assert_grad, assert_loss, check_shard_flow, check_split, ignored_rows, orc, raw_bits, rows_f64,
                      say, to_device_view)
from test_gpu_parity import _g_tensor, _reduced, check_fused

pytestmark = pytest.mark.gpu

SMOOTH = ("all", "others")
REDUCE = ("none", "mean", "sum")


def _upstream(reduce, rows):
    return None if reduce == "none" else 0.7 if reduce == "mean" else 1.0 / 37.0


# ---------------------------------------------------------------------------
# fused call: dtype x layout x smoothing x reduction, ragged 3001-column rows
FUSED = [(dt, sw, sm, red, a) for dt in (torch.float32, torch.bfloat16) for sw in (False, True) for sm in SMOOTH
         for red in REDUCE for a in (0.1, 0.6)]


@pytest.mark.parametrize("dtype,swapped,smoothing,reduce,alpha", FUSED,
                         ids=[f"{'bf16' if f[0] == torch.bfloat16 else 'f32'}-{'sw' if f[1] else 'c'}-{f[2]}-{f[3]}-a{f[4]}"
                              for f in FUSED])
def test_fused_options(dtype, swapped, smoothing, reduce, alpha):
    w = workloads.Workload(93, "options", (3, 8), 3001, dtype, 3.0, 0.2, alpha, reduce != "none", swapped=swapped)
    inp = workloads.generate(w)
    g = _upstream(reduce, w.rows)
    if reduce == "none":
        g = np.linspace(-1.0, 2.0, w.rows)
    check_fused(inp.logits, inp.targets, alpha, reduce, g=g, smoothing=smoothing,
                what=f"options {smoothing} {reduce}")


# split rows (chunks exchange statistics) and the long rows of the main workload
SPLIT = [(dt, V, K, sm, red) for dt in (torch.float32, torch.bfloat16) for V, K in ((8195, 3), (32003, 4))
         for sm in SMOOTH for red in ("none", "sum")]


@pytest.mark.parametrize("dtype,V,K,smoothing,reduce", SPLIT,
                         ids=[f"{'bf16' if s[0] == torch.bfloat16 else 'f32'}-V{s[1]}-K{s[2]}-{s[3]}-{s[4]}"
                              for s in SPLIT])
def test_fused_split_rows_options(dtype, V, K, smoothing, reduce):
    w = workloads.Workload(94, "split-options", (2, 6), V, dtype, 2.0, 0.25, 0.1, reduce != "none")
    inp = workloads.generate(w)
    g = np.linspace(0.5, 1.5, w.rows) if reduce == "none" else 0.25
    check_fused(inp.logits, inp.targets, 0.1, reduce, g=g, split_chunks=K, smoothing=smoothing,
                what=f"split K={K} {smoothing} {reduce}")


@pytest.mark.parametrize("smoothing", SMOOTH)
def test_fused_128000_columns(smoothing):
    """Rows of the main workload's length (auto chunking, BF16 register reuse:
    q_o = 0.1 / 127999 is under the reuse threshold), sum over an external
    count of valid tokens."""
    w = workloads.WORKLOADS[5].scaled(phys=(2, 12), V=128000)
    inp = workloads.generate(w)
    n_global = 3 * (w.rows - w.n_ignored)  # e.g. three data-parallel ranks' valid tokens
    check_fused(inp.logits, inp.targets, w.alpha, "sum", g=1.0 / n_global, smoothing=smoothing,
                what=f"128000 {smoothing} sum/global")


# ---------------------------------------------------------------------------
# forward + backward, and the vocabulary-shard flow
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("smoothing", SMOOTH)
@pytest.mark.parametrize("reduce", REDUCE)
def test_forward_backward_options(dtype, smoothing, reduce):
    w = workloads.Workload(95, "fb-options", (3, 8), 2053, dtype, 2.0, 0.2, 0.3, reduce != "none", swapped=True)
    inp = workloads.generate(w)
    gv = np.linspace(0.5, -0.5, w.rows) if reduce == "none" else 1.3
    check_split(inp.logits, inp.targets, 0.3, reduce, g=gv, smoothing=smoothing,
                what=f"fwd+bwd options {dtype} {smoothing} {reduce}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("smoothing", SMOOTH)
@pytest.mark.parametrize("reduce", ("none", "sum"))
def test_shard_flow_options(dtype, smoothing, reduce):
    V, S = 5003, 4
    w = workloads.Workload(96, "shard-options", (2, 6), V, dtype, 2.0, 0.1, 0.2, reduce != "none", shards=S)
    inp = workloads.generate(w)
    gv = np.linspace(1.0, 2.0, w.rows) if reduce == "none" else 0.9
    check_shard_flow(inp.logits, inp.targets, workloads.shard_bounds(V, S), 0.2, reduce, g=gv, smoothing=smoothing,
                     what=f"shards options {dtype} {smoothing} {reduce}")


# ---------------------------------------------------------------------------
# the external normaliser, the autograd form, degenerate vocabularies
def test_sum_over_external_count_equals_mean_when_count_is_local():
    """sum with g = 1 / n (n the local count) is the mean's gradient: the
    same FP32 scale 1 / n, so the same bits; the loss is the sum."""
    w = workloads.Workload(97, "sum-vs-mean", (4, 16), 4099, torch.bfloat16, 2.0, 0.3, 0.1, True)
    inp = workloads.generate(w)
    n = orc().count_valid(inp.targets)
    xm, _ = check_fused(inp.logits, inp.targets, 0.1, "mean", g=1.0, what="mean")
    xs, ls = check_fused(inp.logits, inp.targets, 0.1, "sum", g=float(np.float32(1.0) / np.float32(n)),
                         what="sum / n")
    assert torch.equal(xm.view(torch.int16), xs.view(torch.int16))


@pytest.mark.parametrize("smoothing", SMOOTH)
@pytest.mark.parametrize("reduce", ("sum", "mean", "none"))
def test_autograd_options(smoothing, reduce):
    x = (torch.randn((2, 9, 4099), generator=torch.Generator().manual_seed(41)) * 2).to(torch.bfloat16)
    t = workloads.random_targets((2, 9), 4099, seed=41, ignore_frac=0.25)
    say(f"[autograd options] {smoothing} {reduce}")
    xd = to_device_view(x).requires_grad_(True)
    td = to_device_view(t)
    loss = vce.parallel_cross_entropy(xd, td, 0.2, reduce, smoothing=smoothing)
    if reduce == "none":
        loss.sum().backward()
    else:
        loss.backward()
    torch.cuda.synchronize()
    o = orc()
    n = o.count_valid(t)
    ref_rows, _ = o.loss_rows(x, t, 0.2, smoothing=smoothing)
    if reduce == "none":
        assert_loss(loss.detach().reshape(-1).cpu().numpy(), ref_rows, "autograd rows")
    else:
        assert_loss([loss.item()], [o.reduce(ref_rows, reduce, n)], f"autograd {reduce}")
    g = np.ones(18) if reduce == "none" else 1.0
    ref = o.grad_rows(x, t, 0.2, reduce_loss=reduce, g=g, n_valid=n, smoothing=smoothing)
    assert xd.grad.data_ptr() == xd.data_ptr()
    assert_grad(rows_f64(xd.grad), ref, torch.bfloat16, f"autograd grad {smoothing} {reduce}")


@pytest.mark.parametrize("V", [1, 2, 3])
def test_tiny_vocabularies_over_the_other_classes(V):
    """V = 2: the other class is a single class getting all of a.  V = 1: only
    a = 0 is defined (plain NLL: loss 0, gradient 0); a > 0 is rejected."""
    g = torch.Generator().manual_seed(V)
    x = (torch.randn((2, 5, V), generator=g) * 2).to(torch.float32)
    t = workloads.random_targets((2, 5), V, seed=V, ignore_frac=0.2)
    alphas = (0.0,) if V == 1 else (0.0, 0.4, 1.0)
    for a in alphas:
        for red in REDUCE:
            check_fused(x, t, a, red, g=None if red == "none" else 0.5, smoothing="others",
                        what=f"V={V} a={a} {red}")
    if V == 1:
        xd, td = to_device_view(x), to_device_view(t)
        with pytest.raises(vce.CeArgumentError):
            vce.ce_fwd_bwd_fused(xd, td, 0.1, True, smoothing="others")
        with pytest.raises(vce.CeArgumentError):
            vce.ce_forward(xd, td, 0.1, True, smoothing="others")


def test_sum_of_no_rows_is_zero():
    x = torch.empty((0, 4, 100), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((0, 4), dtype=torch.int64, device="cuda")
    loss, n = vce.ce_fwd_bwd_fused(x, t, 0.1, "sum")
    l2, _, n2 = vce.ce_forward(x, t, 0.1, "sum")
    torch.cuda.synchronize()
    assert int(n.item()) == 0 and loss.item() == 0.0
    assert int(n2.item()) == 0 and l2.item() == 0.0


def test_sum_all_ignored_is_zero_with_zero_gradient():
    x = (torch.randn((2, 3, 777), generator=torch.Generator().manual_seed(2)) * 2).to(torch.bfloat16)
    t = torch.full((2, 3), -100, dtype=torch.int64)
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.1, "sum", grad_out=torch.tensor([-2.0], device="cuda"),
                                   smoothing="others")
    torch.cuda.synchronize()
    assert int(n.item()) == 0 and loss.item() == 0.0 and not math.isnan(loss.item())
    assert not xd.view(torch.int16).any()

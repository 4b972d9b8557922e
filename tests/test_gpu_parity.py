"""GPU parity of the HIP library against the FP64 oracle, through the C ABI.

Inputs are seeded and synthetic (workloads.py); the oracle reads the exact
bits the GPU consumed.  Oracle-sized cases are compared element by element;
the full-size 128000-column workload is compared in full, in blocks of rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import (assert_grad, assert_loss, check_shard_flow, check_split, ignored_rows, orc, raw_bits, rows_f64,
                      say, to_device_view)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _reduced(reduce) -> bool:
    """True for the mean (True / "mean") and the sum ("sum")."""
    return oracle.reduction_code(reduce) != 0


def _g_tensor(g, reduce):
    if g is None:
        return None
    if _reduced(reduce):
        return torch.tensor([float(g)], dtype=torch.float32, device="cuda")
    return torch.as_tensor(np.asarray(g, dtype=np.float32), device="cuda")


def _s_of(g, reduce, n, N):
    """Per-row gradient scale s_i (for the diagnostic floor)."""
    code = oracle.reduction_code(reduce)
    if code == 1:
        return (1.0 if g is None else float(g)) / max(n, 1)
    if code == 2:
        return 1.0 if g is None else float(g)
    return 1.0


def check_fused(x, t, alpha, reduce, g=None, split_chunks=0, sample=None, what="", diag=True, ws=None,
                smoothing="all"):
    """Run ce_fwd_bwd_fused on a device copy of (x, t) and compare with the oracle.
    Returns the device logits (holding the gradient) and the loss tensor."""
    d0, d1, V = x.shape
    N = d0 * d1
    say(f"[fused] {what} shape={tuple(x.shape)} strides={x.stride()} off={x.storage_offset()} {x.dtype} "
        f"a={alpha} reduce={reduce} smoothing={smoothing} K={split_chunks}")
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = vce.ce_fwd_bwd_fused(xd, td, alpha, reduce, grad_out=_g_tensor(g, reduce), split_chunks=split_chunks,
                                   ws=ws, smoothing=smoothing)
    torch.cuda.synchronize()
    o = orc()
    n_ref = o.count_valid(t)
    assert int(n.item()) == n_ref, (int(n.item()), n_ref)
    rows = np.arange(N) if sample is None else np.asarray(sample, dtype=np.int64)
    ign = set(ignored_rows(t).tolist())
    loss_ref, _ = o.loss_rows(x, t, alpha, rows=rows, smoothing=smoothing)
    if _reduced(reduce):
        if sample is None:
            ref = o.reduce(loss_ref, reduce, n_ref)
            got = float(loss.item())
            if oracle.reduction_code(reduce) == 1 and n_ref == 0:
                assert math.isnan(got) and math.isnan(ref)
            else:
                assert_loss([got], [ref], f"{what} {reduce}")
    else:
        got = loss.cpu().numpy().astype(np.float64)[rows]
        assert_loss(got, loss_ref, what)
        for k, r in enumerate(rows):
            if r in ign:
                assert np.float32(got[k]).view(np.int32) == 0, f"ignored row {r} loss not +0.0"
    g_or = None if g is None else (float(g) if _reduced(reduce) else np.asarray(g, dtype=np.float64))
    grad_ref = o.grad_rows(x, t, alpha, reduce_loss=reduce, g=g_or, rows=rows, n_valid=n_ref, smoothing=smoothing)
    gpu = rows_f64(xd, rows)
    assert_grad(gpu, grad_ref, x.dtype, what)
    if diag and _reduced(reduce) and n_ref > 0:
        # bug-catcher for small s, where the 1e-7 floor hides everything: the
        # floor scaled by s, with 2^-11 |ref| more for BF16 (the kernel may stage
        # exponentials in FP16 between its passes; the official bar above gates)
        s = _s_of(g, reduce, n_ref, N)
        extra = 2.0 ** -11 if x.dtype == torch.bfloat16 else 0.0
        assert_grad(gpu, grad_ref, x.dtype, what + " (floor scaled by s)", floor_scale=min(1.0, abs(s)),
                    extra_rtol=extra)
    ign_rows = [k for k, r in enumerate(rows) if r in ign]
    if ign_rows:
        bits = raw_bits(xd, rows[ign_rows])
        assert not bits.any(), f"{what}: ignored rows not +0.0"
    return xd, loss


# ---------------------------------------------------------------------------
# the five workloads at their full sizes
def test_workload1_split_calls_full():
    w = W[1]
    inp = workloads.generate(w)
    x, t = inp.logits, inp.targets
    N, V = w.rows, w.V
    say(f"[w1] forward + backward {w.name}")
    xd, td = to_device_view(x), to_device_view(t)
    loss, lse, n = vce.ce_forward(xd, td, w.alpha, w.reduce_loss)
    g = torch.ones(N, dtype=torch.float32, device="cuda")
    vce.ce_backward_inplace(xd, td, lse, w.alpha, w.reduce_loss, grad_out=g, n_valid=n)
    torch.cuda.synchronize()
    o = orc()
    assert int(n.item()) == o.count_valid(t) == N - w.n_ignored
    loss_ref, lse_ref = o.loss_rows(x, t, w.alpha)
    assert_loss(loss.cpu().numpy(), loss_ref, "w1 loss")
    kept = t.reshape(-1).numpy() != -100
    assert_loss(lse.cpu().numpy()[kept], lse_ref[kept], "w1 lse")
    assert_grad(rows_f64(xd), o.grad_rows(x, t, w.alpha, g=np.ones(N)), x.dtype, "w1 grad")
    assert not raw_bits(xd, ignored_rows(t)).any()
    # the same calls with the lse_aux hand-off
    check_split(x, t, w.alpha, w.reduce_loss, g=np.ones(N), what="w1", legacy=False)


def test_workload2_swapped_view_full():
    w = W[2]
    inp = workloads.generate(w)
    assert not inp.logits.is_contiguous() and inp.logits.stride() == (w.V, w.phys[1] * w.V, 1)
    check_fused(inp.logits, inp.targets, w.alpha, w.reduce_loss, what=w.name)


def test_workload3_spike_full():
    w = W[3]
    inp = workloads.generate(w)
    xd, loss = check_fused(inp.logits, inp.targets, w.alpha, w.reduce_loss, g=np.ones(w.rows), what=w.name)
    # run-to-run determinism: the same input gives the same bits
    xd2, loss2 = check_fused(inp.logits, inp.targets, w.alpha, w.reduce_loss, g=np.ones(w.rows), what=w.name + " again",
                             sample=[0])
    assert torch.equal(loss, loss2) and torch.equal(xd.view(torch.int16), xd2.view(torch.int16))


def test_workload4_shards_full():
    w = W[4]
    inp = workloads.generate(w)
    x, t = inp.logits, inp.targets
    V, N = w.V, w.rows
    bounds = workloads.shard_bounds(V, w.shards)
    assert [b - a for a, b in bounds] == [16384] * 4
    say(f"[w4] shard flow {w.name}")
    # statistics per shard, combine, backward per shard: loss, n, lse and every
    # gradient element at the stated bar, with no allowance
    stats, loss = check_shard_flow(x, t, bounds, w.alpha, w.reduce_loss, g=np.ones(N), what="w4",
                                   allowance=False)
    o = orc()
    assert o.count_valid(t) == N - w.n_ignored
    kept = t.reshape(-1).numpy() != -100
    # per-shard statistics against the oracle's shard form
    for s, (a, b) in enumerate(bounds):
        st_ref = o.shard_stats(x[..., a:b].contiguous(), t, a, V)
        st = stats[s].cpu().numpy().astype(np.float64)
        assert np.array_equal(st[~kept], np.zeros_like(st[~kept]))
        assert np.array_equal(st[kept, 0], st_ref[kept, 0])        # max is an input value: exact
        assert np.array_equal(st[kept, 2], st_ref[kept, 2])        # target logit: exact
        assert_loss(st[kept, 1], st_ref[kept, 1], "w4 sum-exp")    # relative 1e-4 (values >= 1)
        assert np.all(np.abs(st[kept, 3] - st_ref[kept, 3]) <= 1e-4 * np.maximum(1, np.abs(st_ref[kept, 3])) + 1e-3)
    # the unsharded fused run on a separate copy agrees with the shard flow
    _, loss_full = check_fused(x, t, w.alpha, w.reduce_loss, g=np.ones(N), what="w4 unsharded")
    lf = loss_full.cpu().numpy().astype(np.float64)
    ls = loss.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(ls - lf) <= 1e-4 * np.maximum(1, np.abs(lf)))


def test_workload5_full_size():
    """The 4 x 2048 x 128000 BF16 workload (label smoothing 0.1, mean) in
    full: the fused mean against the oracle's mean over all 8192 rows, every
    row's gradient element by element (blocks of 512 rows), every row's loss
    from an unreduced fused call on a fresh copy, and a second mean call on
    another copy bit for bit equal to the first."""
    w = W[5]
    say(f"[w5] generating {w.name}")
    inp = workloads.generate(w)
    x, t = inp.logits, inp.targets
    N, V = w.rows, w.V
    o = orc()
    n_ref = o.count_valid(t)
    assert n_ref == N - w.n_ignored
    say("[w5] fused mean at full size")
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = vce.ce_fwd_bwd_fused(xd, td, w.alpha, w.reduce_loss)
    torch.cuda.synchronize()
    assert int(n.item()) == n_ref
    ref_rows, _ = o.loss_rows(x, t, w.alpha)
    assert_loss([loss.item()], [o.mean_loss(ref_rows, n_ref)], "w5 mean")
    s = 1.0 / n_ref
    ign = set(ignored_rows(t).tolist())
    B = 512
    for r0 in range(0, N, B):
        rows = np.arange(r0, min(N, r0 + B))
        say(f"[w5] gradient rows {r0}..{rows[-1]}")
        ref = o.grad_rows(x, t, w.alpha, reduce_loss=w.reduce_loss, rows=rows, n_valid=n_ref)
        gpu = rows_f64(xd, rows)
        assert_grad(gpu, ref, x.dtype, f"w5 rows {r0}+")
        # the floor scaled by s (the stated 1e-7 floor hides most |ref| at s = 1/7782), with the FP16
        # staging's 2^-11 relative error on top
        assert_grad(gpu, ref, x.dtype, f"w5 rows {r0}+ (floor scaled by s)", floor_scale=s, extra_rtol=2.0 ** -11)
        mine = [k for k, r in enumerate(rows) if r in ign]
        if mine:
            assert not raw_bits(xd, rows[mine]).any(), "ignored rows must be +0.0"
        del ref, gpu
    say("[w5] second fused mean on a fresh copy (determinism)")
    xd2 = to_device_view(x)
    loss2, _ = vce.ce_fwd_bwd_fused(xd2, td, w.alpha, w.reduce_loss)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)
    assert torch.equal(xd.view(torch.int16), xd2.view(torch.int16))
    del xd2
    say("[w5] unreduced fused call on a fresh copy: every row's loss")
    xd3 = to_device_view(x)
    rl, _ = vce.ce_fwd_bwd_fused(xd3, td, w.alpha, False)
    torch.cuda.synchronize()
    got = rl.cpu().numpy().astype(np.float64)
    assert_loss(got, ref_rows, "w5 per-row losses")
    assert not got[sorted(ign)].view(np.int64).any(), "ignored rows' loss must be +0.0"


# ---------------------------------------------------------------------------
# the same recipes at oracle sizes (several tiles, ragged tails)
SCALED = [
    ("w1", W[1].scaled(phys=(2, 40), V=4099)),
    ("w2", W[2].scaled(phys=(4, 24), V=8195)),
    ("w3", W[3].scaled(phys=(2, 40), V=31999)),
    ("w5", W[5].scaled(phys=(2, 12), V=128003)),
    ("w5_fp32", W[5].scaled(phys=(2, 6), V=70001)),
]


@pytest.mark.parametrize("name,w", SCALED, ids=[s[0] for s in SCALED])
def test_scaled_workloads_fused(name, w):
    inp = workloads.generate(w)
    x = inp.logits if w.dtype != torch.float32 or name != "w5_fp32" else inp.logits
    if name == "w5_fp32":
        x = inp.logits.to(torch.float32)
    g = None if w.reduce_loss else np.linspace(0.25, 1.75, w.rows)
    check_fused(x, inp.targets, w.alpha, w.reduce_loss, g=g, what=name)


# ---------------------------------------------------------------------------
# off-config matrix: dtype x reduce x layout x smoothing x ignore density
MATRIX = [(dt, red, sw, a, p) for dt in (torch.float32, torch.bfloat16) for red in (False, True)
          for sw in (False, True) for a in (0.0, 0.1) for p in (0.0, 0.05, 1.0)]


@pytest.mark.parametrize("dtype,reduce,swapped,alpha,ignore", MATRIX,
                         ids=[f"{'bf16' if m[0] == torch.bfloat16 else 'f32'}-r{int(m[1])}-{'sw' if m[2] else 'c'}"
                              f"-a{m[3]}-i{m[4]}" for m in MATRIX])
def test_matrix_fused(dtype, reduce, swapped, alpha, ignore):
    w = workloads.Workload(90, "matrix", (3, 8), 3001, dtype, 3.0, ignore, alpha, reduce, swapped=swapped)
    inp = workloads.generate(w)
    g = 0.6 if reduce else np.linspace(-1.0, 2.0, w.rows)
    check_fused(inp.logits, inp.targets, alpha, reduce, g=g, what="matrix")


@pytest.mark.parametrize("dtype,reduce,swapped,alpha", [(d, r, s, a) for d in (torch.float32, torch.bfloat16)
                                                        for r in (False, True) for s in (False, True)
                                                        for a in (0.0, 0.1)])
def test_matrix_forward_backward(dtype, reduce, swapped, alpha):
    w = workloads.Workload(91, "fb", (3, 8), 2053, dtype, 2.0, 0.2, alpha, reduce, swapped=swapped)
    inp = workloads.generate(w)
    gv = 1.3 if reduce else np.linspace(0.5, -0.5, w.rows)
    check_split(inp.logits, inp.targets, alpha, reduce, g=gv,
                what=f"fwd+bwd {dtype} reduce={reduce} swapped={swapped} a={alpha}")


# ---------------------------------------------------------------------------
# ragged and misaligned rows
# 70001 columns: rows of several backward items (BF16 3, FP32 5) with a head and a tail when offset
RAGGED = [(dt, V, off) for dt in (torch.float32, torch.bfloat16)
          for V in (1, 2, 7, 8, 9, 15, 17, 33, 1000, 4095, 32003, 70001) for off in (0, 1)]


@pytest.mark.parametrize("dtype,V,offset", RAGGED, ids=[f"{'bf16' if r[0] == torch.bfloat16 else 'f32'}-V{r[1]}-off{r[2]}"
                                                         for r in RAGGED])
def test_ragged_and_misaligned(dtype, V, offset):
    g = torch.Generator().manual_seed(V * 7 + offset)
    A, B = 3, 5
    storage = (torch.randn(A * B * V + offset, generator=g) * 2).to(dtype)
    x = storage[offset:].view(A, B, V)
    t = workloads.random_targets((A, B), V, seed=V + 11, ignore_frac=0.2)
    assert x.storage_offset() == offset
    check_fused(x, t, 0.1, False, g=np.linspace(0.5, 1.5, A * B), what=f"ragged V={V} off={offset}")
    # forward + backward on the same layout
    check_split(x, t, 0.1, False, what=f"ragged V={V} off={offset}")


# ---------------------------------------------------------------------------
# rows split over cooperating workgroups
SPLITS = [(dt, V, K, off) for dt in (torch.float32, torch.bfloat16) for V, K in ((4096, 2), (4096, 3), (4096, 7),
                                                                                  (32003, 4), (2048, 64), (130, 5))
          for off in (0, 3)]


@pytest.mark.parametrize("dtype,V,K,offset", SPLITS,
                         ids=[f"{'bf16' if s[0] == torch.bfloat16 else 'f32'}-V{s[1]}-K{s[2]}-off{s[3]}" for s in SPLITS])
def test_forced_split(dtype, V, K, offset):
    g = torch.Generator().manual_seed(V + K)
    A, B = 2, 9
    storage = (torch.randn(A * B * V + offset, generator=g) * 3).to(dtype)
    x = storage[offset:].view(A, B, V)
    t = workloads.random_targets((A, B), V, seed=K, ignore_frac=0.15)
    for reduce in (False, True):
        check_fused(x, t, 0.1, reduce, g=1.0 if reduce else None, split_chunks=K, what=f"split V={V} K={K}")
    # the exchange never gave up
    xd, td = to_device_view(x), to_device_view(t)
    ws = torch.empty(vce.ce_workspace_bytes(xd, 0.1, True, split_chunks=K), dtype=torch.uint8, device="cuda")
    vce.ce_fwd_bwd_fused(xd, td, 0.1, True, ws=ws, split_chunks=K)
    vce.ce_workspace_check(ws)


def test_split_equals_unsplit_bits_of_loss_close():
    w = W[3].scaled(phys=(2, 8), V=32000)
    inp = workloads.generate(w)
    _, l1 = check_fused(inp.logits, inp.targets, 0.0, False, what="K=1")
    _, l4 = check_fused(inp.logits, inp.targets, 0.0, False, split_chunks=4, what="K=4")
    a, b = l1.cpu().numpy().astype(np.float64), l4.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a - b) <= 1e-5 * np.maximum(1, np.abs(a)))


# ---------------------------------------------------------------------------
# uneven vocabulary shards (ceil(V / S) columns per shard)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,S", [(1001, 4), (65, 3), (5003, 7), (16384 * 4 + 5, 4)])
@pytest.mark.parametrize("reduce", [False, True])
def test_uneven_shards(dtype, V, S, reduce):
    w = workloads.Workload(92, "shards", (2, 6), V, dtype, 2.0, 0.1, 0.1, reduce, shards=S)
    inp = workloads.generate(w)
    gv = 0.9 if reduce else np.linspace(1.0, 2.0, w.rows)
    check_shard_flow(inp.logits, inp.targets, workloads.shard_bounds(V, S), 0.1, reduce, g=gv,
                     what=f"shards V={V} S={S} {dtype} reduce={reduce}")


# ---------------------------------------------------------------------------
# degenerate cases
def test_empty_rows():
    x = torch.empty((0, 4, 100), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((0, 4), dtype=torch.int64, device="cuda")
    loss, n = vce.ce_fwd_bwd_fused(x, t, 0.1, True)
    loss0, n0 = vce.ce_fwd_bwd_fused(x, t, 0.1, False)
    l2, lse2, n2 = vce.ce_forward(x, t, 0.0, True)
    torch.cuda.synchronize()
    assert int(n.item()) == 0 and math.isnan(loss.item()) and loss0.numel() == 0
    assert int(n2.item()) == 0 and math.isnan(l2.item())


def test_all_ignored_mean_is_nan_and_grads_zero():
    x = (torch.randn((2, 3, 777), generator=torch.Generator().manual_seed(1)) * 2).to(torch.bfloat16)
    t = torch.full((2, 3), -100, dtype=torch.int64)
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.1, True, grad_out=torch.tensor([-2.0], device="cuda"))
    torch.cuda.synchronize()
    assert int(n.item()) == 0 and math.isnan(loss.item())
    assert not xd.view(torch.int16).any()


def test_negative_upstream_gradient_keeps_ignored_rows_plus_zero():
    w = workloads.Workload(93, "neg", (2, 8), 1500, torch.float32, 2.0, 0.25, 0.1, False)
    inp = workloads.generate(w)
    check_fused(inp.logits, inp.targets, 0.1, False, g=-np.ones(w.rows), what="negative g")


def test_custom_ignore_index_and_invalid_targets_give_nan_rows():
    x = (torch.randn((1, 6, 300), generator=torch.Generator().manual_seed(4)) * 2).to(torch.float32)
    t = torch.tensor([[5, -1, 299, 300, -7, 0]])  # -1 ignored; 300 and -7 out of range
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.0, False, ignore_idx=-1)
    torch.cuda.synchronize()
    assert int(n.item()) == 5
    lv = loss.cpu().numpy()
    assert lv[1] == 0.0 and np.isnan(lv[3]) and np.isnan(lv[4])
    gr = rows_f64(xd)
    assert np.isnan(gr[3]).all() and np.isnan(gr[4]).all() and not gr[1].any()
    o = orc()
    xs, ts = x[:, [0, 2, 5]], t[:, [0, 2, 5]]
    ref, _ = o.loss_rows(xs.contiguous(), ts.contiguous(), 0.0)
    assert_loss(lv[[0, 2, 5]], ref, "valid rows next to invalid ones")


def test_uniform_logits_closed_form_at_128000():
    V = 128000
    x = torch.full((1, 4, V), 100.0, dtype=torch.bfloat16)
    t = torch.tensor([[0, V - 1, 64000, 77]])
    xd, td = to_device_view(x), to_device_view(t)
    loss, _ = vce.ce_fwd_bwd_fused(xd, td, 0.1, False)
    torch.cuda.synchronize()
    assert np.all(np.abs(loss.cpu().numpy() - math.log(V)) <= 1e-4 * math.log(V))
    gr = rows_f64(xd)
    for k in range(4):
        ref = 0.9 * (1.0 / V - (np.arange(V) == int(t[0, k])))
        assert_grad(gr[k], ref, torch.bfloat16, "uniform grad")


def test_confident_rows():
    """Rows whose target holds almost all the probability (p_t close to 1)."""
    for dtype in (torch.bfloat16, torch.float32):
        g = torch.Generator().manual_seed(17)
        x = torch.randn((2, 8, 5000), generator=g)
        t = torch.randint(0, 5000, (2, 8), generator=g)
        for k in range(16):
            x.view(16, 5000)[k, t.view(-1)[k]] = 9.0 + k  # p_t from ~0.6 to ~1 - 1e-6
        check_fused(x.to(dtype), t, 0.0, False, what=f"confident {dtype}")
        check_fused(x.to(dtype), t, 0.1, True, what=f"confident smoothed {dtype}")


# ---------------------------------------------------------------------------
# the issue #29 interface and streams
def test_parallel_cross_entropy_interface():
    w = W[2].scaled(phys=(4, 16), V=8192)
    inp = workloads.generate(w)
    xd, td = to_device_view(inp.logits), to_device_view(inp.targets)
    loss = vce.parallel_cross_entropy(xd, td, label_smoothing=0.1, reduce_loss=False)
    torch.cuda.synchronize()
    assert loss.shape == td.shape and loss.dtype == torch.float32
    o = orc()
    ref, _ = o.loss_rows(inp.logits, inp.targets, 0.1)
    assert_loss(loss.reshape(-1).cpu().numpy(), ref, "interface loss")
    assert_grad(rows_f64(xd), o.grad_rows(inp.logits, inp.targets, 0.1), torch.bfloat16, "interface grad")
    with pytest.raises(NotImplementedError):
        vce.parallel_cross_entropy(xd, td, dist_process_group=object())
    with pytest.raises(vce.CeArgumentError):
        vce.parallel_cross_entropy(xd.to(torch.float16), td)


def test_runs_on_the_callers_stream():
    w = W[3].scaled(phys=(2, 16), V=32000)
    inp = workloads.generate(w)
    s = torch.cuda.Stream()
    xd, td = to_device_view(inp.logits), to_device_view(inp.targets)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.0, False)
    s.synchronize()
    ref, _ = orc().loss_rows(inp.logits, inp.targets, 0.0)
    assert_loss(loss.cpu().numpy(), ref, "side stream")

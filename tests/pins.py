"""Pins of the FP64 oracle against facts fixed outside it.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix.  They
run against the real oracle (tests/test_oracle_pins.py) and against copies of
it with planted mistakes (tests/test_oracle_mutants.py), where at least one
pin must fail for every mistake.

What each pin rests on:
  * brute force -- the unfused softmax -> log -> NLL chain of the CANN ops-nn
    fusion page ("standard approach: three kernels"), run in 50-digit decimal,
    with either smoothed target distribution;
  * closed form -- uniform logits give softmax 1/V, so the loss is ln V for
    any smoothing and any target, and the gradient is s (1/V - q_j);
  * the ops-nn page's worked number ("pitfall 1"): logits all 100, V = 32000,
    lse = 100 + ln 32000, printed as 110.4 (tests/golden/p4_uniform_lse.json);
  * library special case -- torch's float64 F.cross_entropy with
    ignore_index and label_smoothing (the precision baseline named on the
    TransformerEngineNPU issue #29 page, section 4) and its autograd gradient,
    for the none, mean and sum reductions.  Smoothing a over the V - 1 other
    classes (the ops-nn page's kernel) gives the target 1 - a and every other
    class a / (V - 1); torch's smoothing a' over all V classes gives the same
    distribution when a' = a V / (V - 1), so torch pins that convention too;
  * finite differences -- the gradient is the derivative of the loss;
  * invariants -- a row shift leaves loss and gradient unchanged, and
    non-ignored gradient rows sum to zero;
  * sharded == unsharded -- the vocabulary-parallel combine (hyper-parallel
    issue #269 page, section 3.1) is an identity.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: max err {err.max():.3e} (worst at {np.unravel_index(np.argmax(err - bound), err.shape)})"


def _tiny_case(seed, N, V, dtype, alpha, ignore_frac=0.25, swapped=False):
    g = torch.Generator().manual_seed(seed)
    A, B = (2, N // 2) if N % 2 == 0 else (1, N)
    phys = (torch.randn((A, B, V), generator=g) * 3).to(dtype)
    t = torch.randint(0, V, (A, B), generator=g)
    k = int(round(ignore_frac * A * B))
    if k:
        t.view(-1)[torch.randperm(A * B, generator=g)[:k]] = workloads.IGNORE_IDX
    if swapped:
        return phys.transpose(0, 1), t.transpose(0, 1)
    return phys, t


def _rows_of(x):
    """Logical rows as lists of Python floats (exact values of the stored bits)."""
    d0, d1, V = x.shape
    xd = x.to(torch.float64)
    return [[float(v) for v in xd[i0, i1]] for i0 in range(d0) for i1 in range(d1)]


def _targets_of(t):
    d0, d1 = t.shape
    return [int(t[i0, i1]) for i0 in range(d0) for i1 in range(d1)]


# ----------------------------------------------------------------------------
def pin_brute_force(orc):
    """Oracle loss == 50-digit softmax -> log -> NLL, tiny inputs, all layouts,
    both smoothing conventions (over the other classes needs V >= 2 once a > 0)."""
    cases = 0
    for seed, (N, V) in enumerate([(4, 1), (4, 2), (4, 5), (6, 8), (3, 7), (8, 16)]):
        for dtype in (torch.float32, torch.bfloat16):
            for alpha in (0.0, 0.1, 0.7):
                for swapped in (False, True):
                    for smoothing in ("all", "others"):
                        x, t = _tiny_case(100 + seed, N, V, dtype, alpha, swapped=swapped)
                        if smoothing == "others" and V == 1 and alpha > 0:
                            try:
                                orc.loss_rows(x, t, alpha=alpha, smoothing=smoothing)
                            except oracle.OracleError:
                                continue
                            raise AssertionError("a > 0 over the other classes of a 1-class row must be rejected")
                        loss, _ = orc.loss_rows(x, t, alpha=alpha, smoothing=smoothing)
                        ref = brute.loss_rows(_rows_of(x), _targets_of(t), alpha=alpha, smoothing=smoothing)
                        _close(loss, [float(r) for r in ref], 1e-12, 1e-15,
                               f"brute N={N} V={V} {dtype} a={alpha} {smoothing}")
                        cases += 1
    assert cases == 136


def pin_closed_form_uniform(orc):
    """Uniform logits: loss = ln V for every smoothing; grad = s (1/V - q_j),
    which is s (1-a)(1/V - onehot) over all classes and s (1/V - (1-a)) at the
    target, s (1/V - a/(V-1)) elsewhere over the other classes.

    c = 1000 overflows exp() in FP64 unless the row maximum is taken out first."""
    for V in (1, 7, 4096, 32000):
        for c in (0.0, -37.5, 100.0, 1000.0):
            for alpha in (0.0, 0.1, 0.5):
                for smoothing in ("all", "others"):
                    if smoothing == "others" and V == 1 and alpha > 0:
                        continue
                    x = torch.full((1, 3, V), c, dtype=torch.float32)
                    t = torch.tensor([[0, V - 1, V // 2]])
                    loss, lse = orc.loss_rows(x, t, alpha=alpha, smoothing=smoothing)
                    _close(loss, [math.log(V)] * 3, 1e-12, 1e-12, f"ln V, V={V} c={c} a={alpha} {smoothing}")
                    _close(lse, [c + math.log(V)] * 3, 1e-13, 1e-12, f"lse V={V} c={c}")
                    if V <= 4096:
                        g = np.array([0.5, 2.0, -1.0])
                        grad = orc.grad_rows(x, t, alpha=alpha, g=g, smoothing=smoothing)
                        ref = np.empty_like(grad)
                        for k in range(3):
                            onehot = np.arange(V) == int(t[0, k])
                            if smoothing == "all":
                                ref[k] = g[k] * (1 - alpha) * (1.0 / V - onehot)
                            else:
                                other = alpha / (V - 1) if V > 1 else 0.0
                                ref[k] = g[k] * (1.0 / V - np.where(onehot, 1 - alpha, other))
                        _close(grad, ref, 1e-12, 1e-15, f"uniform grad V={V} c={c} a={alpha} {smoothing}")


def pin_golden_p4_worked_lse(orc):
    """The ops-nn page's worked value: all logits 100, V = 32000, lse ~ 110.4."""
    with open(os.path.join(GOLDEN, "p4_uniform_lse.json")) as f:
        gold = json.load(f)
    V, c = gold["V"], gold["logit"]
    x = torch.full((1, 1, V), c, dtype=torch.float32)
    t = torch.tensor([[gold["target"]]])
    _, lse = orc.loss_rows(x, t)
    printed = gold["lse_printed"]
    assert abs(lse[0] - printed) <= gold["printed_half_unit"], (lse[0], printed)
    assert abs((lse[0] - c) - gold["log_v_printed"]) <= gold["printed_half_unit"]


def pin_golden_p4_other_class_share(orc):
    """The ops-nn page's per-class smoothing share a / (V - 1) at a = 0.1,
    V = 32000, printed as about 3.1e-6: with the target holding nearly all the
    probability (other classes' p ~ e^-60), every other class's gradient is
    minus that share."""
    with open(os.path.join(GOLDEN, "p4_smoothing_other_class.json")) as f:
        gold = json.load(f)
    V, alpha = gold["V"], gold["alpha"]
    x = torch.zeros((1, 1, V), dtype=torch.float32)
    x[0, 0, 7] = 60.0
    t = torch.tensor([[7]])
    grad = orc.grad_rows(x, t, alpha=alpha, smoothing="others")[0]
    others = np.delete(grad, 7)
    assert np.all(np.abs(-others - gold["share_printed"]) <= gold["printed_half_unit"]), others[:3]
    _close(-others, np.full(V - 1, alpha / (V - 1)), 1e-12, 0.0, "other-class share")


def _torch_smoothing(alpha, V, smoothing):
    """torch's all-class smoothing that puts the same mass on every class."""
    return alpha if smoothing == "all" else alpha * V / (V - 1)


def pin_torch_cross_entropy(orc):
    """Oracle loss, mean, sum and gradient == torch float64 F.cross_entropy + autograd."""
    for seed, (N, V) in enumerate([(8, 3), (12, 50), (6, 257), (16, 1000)]):
        for dtype in (torch.float32, torch.bfloat16):
            for alpha in (0.0, 0.1, 0.3):
                for swapped in (False, True):
                    for smoothing in ("all", "others"):
                        x, t = _tiny_case(200 + seed, N, V, dtype, alpha, ignore_frac=0.2, swapped=swapped)
                        d0, d1, _ = x.shape
                        a_t = _torch_smoothing(alpha, V, smoothing)
                        what = f"{N}x{V} a={alpha} {smoothing}"
                        xd = x.to(torch.float64).reshape(d0 * d1, V).clone().requires_grad_(True)
                        tf = t.reshape(d0 * d1)
                        ref = F.cross_entropy(xd, tf, ignore_index=-100, label_smoothing=a_t, reduction="none")
                        loss, _ = orc.loss_rows(x, t, alpha=alpha, smoothing=smoothing)
                        _close(loss, ref.detach().numpy(), 1e-12, 1e-14, f"torch loss {what}")
                        g = torch.linspace(-1.5, 2.0, d0 * d1, dtype=torch.float64)
                        (gx,) = torch.autograd.grad(ref, xd, g)
                        grad = orc.grad_rows(x, t, alpha=alpha, g=g.numpy(), smoothing=smoothing)
                        _close(grad, gx.numpy(), 1e-11, 1e-15, f"torch grad (none) {what}")
                        n = orc.count_valid(t)
                        # mean over non-ignored rows and sum over rows, upstream scalar g = 0.75
                        for red in ("mean", "sum"):
                            xm = x.to(torch.float64).reshape(d0 * d1, V).clone().requires_grad_(True)
                            refm = F.cross_entropy(xm, tf, ignore_index=-100, label_smoothing=a_t, reduction=red)
                            _close([orc.reduce(loss, red, n)], [float(refm.detach())], 1e-12, 1e-14, f"torch {red}")
                            (gm,) = torch.autograd.grad(refm, xm, torch.tensor(0.75, dtype=torch.float64))
                            gradm = orc.grad_rows(x, t, alpha=alpha, reduce_loss=red, g=0.75, smoothing=smoothing)
                            _close(gradm, gm.numpy(), 1e-11, 1e-15, f"torch grad ({red}) {what}")
                        gradb = orc.grad_rows(x, t, alpha=alpha, reduce_loss=True, g=0.75, smoothing=smoothing)
                        _close(gradb, orc.grad_rows(x, t, alpha=alpha, reduce_loss="mean", g=0.75,
                                                    smoothing=smoothing), 0, 0, "reduce_loss=True is the mean")


def pin_mean_all_ignored_is_nan(orc):
    """Mean over zero non-ignored rows is 0/0 = NaN, as torch's mean reduction."""
    x = torch.randn((2, 3, 5), generator=torch.Generator().manual_seed(7))
    t = torch.full((2, 3), -100)
    loss, _ = orc.loss_rows(x, t)
    n = orc.count_valid(t)
    ref = F.cross_entropy(x.double().reshape(6, 5), t.reshape(6), ignore_index=-100, reduction="mean")
    assert n == 0 and math.isnan(orc.mean_loss(loss, n)) and math.isnan(float(ref))
    assert np.all(loss == 0.0)


def pin_finite_differences(orc):
    """grad == central differences of sum_i g_i loss_i (and of g * mean, g * sum),
    for both smoothing conventions.

    Logits sit on the 2^-10 grid and the step is 2^-10, so x +- h is exact in
    FP32 and the only error is the O(h^2) truncation."""
    h = 2.0 ** -10
    for alpha in (0.0, 0.2):
        for smoothing in ("all", "others"):
            for red in ("none", "mean", "sum"):
                g = torch.Generator().manual_seed(31 + len(red))
                x = (torch.randint(-2048, 2048, (2, 2, 6), generator=g).double() * h).float()
                t = torch.tensor([[1, -100], [5, 0]])
                gr = np.array([0.7, -1.3, 2.0, 0.4])
                gs = 1.7
                n = orc.count_valid(t)

                def objective(xx):
                    loss, _ = orc.loss_rows(xx, t, alpha=alpha, smoothing=smoothing)
                    return float(np.dot(gr, loss)) if red == "none" else gs * orc.reduce(loss, red, n)

                grad = orc.grad_rows(x, t, alpha=alpha, reduce_loss=red, g=gr if red == "none" else gs,
                                     smoothing=smoothing)
                fd = np.zeros_like(grad)
                for r in range(4):
                    i0, i1 = divmod(r, 2)
                    for j in range(6):
                        xp, xm = x.clone(), x.clone()
                        xp[i0, i1, j] += h
                        xm[i0, i1, j] -= h
                        fd[r, j] = (objective(xp) - objective(xm)) / (2 * h)
                _close(grad, fd, 1e-4, 1e-7, f"finite differences a={alpha} {smoothing} {red}")


def pin_shift_invariance(orc):
    """x -> x + c per row leaves loss and gradient unchanged (grid-exact shift)."""
    for dtype in (torch.float32, torch.bfloat16):
        x = workloads.grid_logits((3, 4, 37), dtype, seed=5)
        t = workloads.random_targets((3, 4), 37, seed=6, ignore_frac=0.25)
        xs = (x.double() + 4.0).to(dtype)
        assert torch.equal(xs.double() - 4.0, x.double())
        for alpha in (0.0, 0.3):
            for smoothing in ("all", "others"):
                l0, _ = orc.loss_rows(x, t, alpha=alpha, smoothing=smoothing)
                l1, _ = orc.loss_rows(xs, t, alpha=alpha, smoothing=smoothing)
                _close(l1, l0, 1e-12, 1e-13, f"shift loss {smoothing}")
                g0 = orc.grad_rows(x, t, alpha=alpha, smoothing=smoothing)
                g1 = orc.grad_rows(xs, t, alpha=alpha, smoothing=smoothing)
                _close(g1, g0, 1e-11, 1e-15, f"shift grad {smoothing}")


def pin_grad_rows_sum_to_zero(orc):
    """sum_j grad_ij = s (1 - (1-a) - a) = 0 for kept rows; ignored rows are exactly 0."""
    inp = workloads.generate(workloads.WORKLOADS[2].scaled(phys=(4, 8), V=300))
    for alpha in (0.0, 0.1):
        for red in ("none", "mean", "sum"):
            for smoothing in ("all", "others"):
                grad = orc.grad_rows(inp.logits, inp.targets, alpha=alpha, reduce_loss=red,
                                     g=None if red == "none" else 0.9, smoothing=smoothing)
                t = inp.targets.reshape(-1).numpy()
                kept = t != -100
                assert np.all(grad[~kept] == 0.0)
                sums = grad[kept].sum(axis=1)
                scale = np.abs(grad[kept]).sum(axis=1)
                assert np.all(np.abs(sums) <= 1e-13 * np.maximum(scale, 1e-300)), np.abs(sums).max()


def pin_sharded_equals_unsharded(orc):
    """Per-shard (m, d, y, r) then combine == the unsharded loss, lse and grad."""
    for V, shards in ((1000, 4), (1001, 4), (65, 3), (5, 5)):
        w = workloads.WORKLOADS[4].scaled(phys=(2, 5), V=V)
        inp = workloads.generate(w)
        x, t = inp.logits, inp.targets
        bounds = workloads.shard_bounds(V, shards)
        assert bounds[-1][1] == V
        for alpha in (0.0, 0.1):
            for smoothing in ("all", "others"):
                full_loss, full_lse = orc.loss_rows(x, t, alpha=alpha, smoothing=smoothing)
                stats = np.stack([orc.shard_stats(x[..., a:b].contiguous(), t, a, V) for a, b in bounds])
                loss, lse = orc.shard_combine(stats, t, V, alpha=alpha, smoothing=smoothing)
                kept = t.reshape(-1).numpy() != -100
                _close(loss, full_loss, 1e-12, 1e-13, f"shard loss V={V} S={shards} {smoothing}")
                _close(lse[kept], full_lse[kept], 1e-13, 1e-13, "shard lse")
                for red, g in (("none", np.linspace(0.5, 1.5, 10)), ("sum", 0.6)):
                    full_grad = orc.grad_rows(x, t, alpha=alpha, g=g, reduce_loss=red, smoothing=smoothing)
                    parts = [orc.shard_grad(x[..., a:b].contiguous(), t, a, V, np.where(kept, lse, 0.0),
                                            alpha=alpha, g=g, reduce_loss=red, smoothing=smoothing)
                             for a, b in bounds]
                    _close(np.concatenate(parts, axis=1), full_grad, 1e-12, 1e-16,
                           f"shard grad V={V} S={shards} {smoothing} {red}")


def pin_count_and_rows(orc):
    """n equals the rows the generator kept, and sampled rows equal full rows."""
    for k in (1, 2, 3, 4):
        w = workloads.WORKLOADS[k].scaled(phys=(2, 16), V=64)
        inp = workloads.generate(w)
        assert orc.count_valid(inp.targets) == w.rows - w.n_ignored
        rows = np.array([w.rows - 1, 0, 7, 3])
        full, _ = orc.loss_rows(inp.logits, inp.targets, alpha=w.alpha)
        part, _ = orc.loss_rows(inp.logits, inp.targets, alpha=w.alpha, rows=rows)
        assert np.array_equal(part, full[rows])


def pin_masked_logits(orc):
    """Logits of -inf (masked classes) against torch float64: the loss is finite
    where the smoothing gives those classes no weight (0 log 0 = 0) and +inf
    where it does, or where the target itself is masked; gradients are finite.
    Loss and lse also through the shard form."""
    for dtype in (torch.float32, torch.bfloat16):
        g = torch.Generator().manual_seed(91)
        x = (torch.randn((1, 6, 13), generator=g) * 2).to(dtype)
        x[0, :, 3] = -float("inf")
        x[0, 1, 7:11] = -float("inf")
        t = torch.tensor([[0, 2, 5, -100, 3, 12]])  # row 4's target is masked
        for smoothing in ("all", "others"):
            for alpha in (0.0, 0.2):
                a_t = _torch_smoothing(alpha, 13, smoothing)
                xd = x.to(torch.float64).reshape(6, 13).clone().requires_grad_(True)
                ref = F.cross_entropy(xd, t.reshape(6), ignore_index=-100, label_smoothing=a_t, reduction="none")
                (gx,) = torch.autograd.grad(ref.masked_fill(~torch.isfinite(ref), 0.0).sum(), xd)
                loss, _ = orc.loss_rows(x, t, alpha, smoothing=smoothing)
                r = ref.detach().numpy()
                what = f"masked {dtype} {smoothing} a={alpha}"
                assert np.array_equal(np.isinf(loss), np.isinf(r)), (what, loss, r)
                fin = np.isfinite(r)
                _close(loss[fin], r[fin], 1e-12, 1e-14, what + " loss")
                # the gradient of rows whose loss is finite (torch's own grad of an inf row is its finite limit too)
                grad = orc.grad_rows(x, t, alpha, smoothing=smoothing, g=np.ones(6))
                _close(grad[fin], gx.numpy()[fin], 1e-11, 1e-15, what + " grad")
                assert np.all(np.isfinite(grad))
                stats = orc.shard_stats(x, t, 0, 13)[None]
                sl, _ = orc.shard_combine(stats, t, 13, alpha, smoothing=smoothing)
                assert np.array_equal(np.isinf(sl), np.isinf(r)), (what, sl, r)
                _close(sl[fin], r[fin], 1e-12, 1e-14, what + " shard loss")


def _linear_case(seed, N, D, V, dtype, ignore=2):
    g = torch.Generator().manual_seed(seed)
    h = (torch.randn((N, D), generator=g)).to(dtype)
    w = (torch.randn((V, D), generator=g) * (2.0 / math.sqrt(D))).to(dtype)
    t = torch.randint(0, V, (N,), generator=g)
    t[torch.randperm(N, generator=g)[:ignore]] = -100
    return h, w, t


def pin_linear_identity_head(orc):
    """Head = identity (D = V): the logits are h itself, so the loss and dh are
    the cross-entropy oracle's loss and gradient (pinned above), and dW = G^T h."""
    for dtype in (torch.float32, torch.bfloat16):
        for smoothing in ("all", "others"):
            for red in ("none", "mean", "sum"):
                g = torch.Generator().manual_seed(61)
                V = 9
                h = (torch.randn((6, V), generator=g) * 2).to(dtype)
                w = torch.eye(V, dtype=dtype)
                t = torch.tensor([0, 8, -100, 3, 3, 5])
                gg = np.linspace(0.5, 1.5, 6) if red == "none" else 0.7
                loss, dh, dw = orc.linear_ce(h, w, t, 0.2, reduce_loss=red, g=gg, smoothing=smoothing)
                x3, t2 = h.view(1, 6, V), t.view(1, 6)
                ref_loss, _ = orc.loss_rows(x3, t2, 0.2, smoothing=smoothing)
                ref_g = orc.grad_rows(x3, t2, 0.2, reduce_loss=red, g=gg, smoothing=smoothing)
                _close(loss, ref_loss, 1e-13, 1e-15, f"identity head loss {dtype} {smoothing} {red}")
                _close(dh, ref_g, 1e-13, 1e-16, "identity head dh")
                _close(dw, ref_g.T @ h.double().numpy(), 1e-12, 1e-16, "identity head dW = G^T h")


def pin_linear_torch(orc):
    """Loss, dh and dW == torch float64: logits h W^T rounded as the library
    materialises them (FP32, then BF16 for BF16 inputs, nearest even), then
    F.cross_entropy with autograd on the rounded logits, dh = G W, dW = G^T h."""
    for dtype in (torch.float32, torch.bfloat16):
        for N, D, V in ((5, 7, 11), (8, 16, 33)):
            for smoothing in ("all", "others"):
                for red in ("none", "mean", "sum"):
                    h, w, t = _linear_case(70 + N + V, N, D, V, dtype)
                    x = (h.double() @ w.double().T).float()
                    if dtype == torch.bfloat16:
                        x = x.to(torch.bfloat16)
                    x = x.double().requires_grad_(True)
                    a_t = _torch_smoothing(0.1, V, smoothing)
                    ref = F.cross_entropy(x, t, ignore_index=-100, label_smoothing=a_t, reduction=red)
                    if red == "none":
                        gg = torch.linspace(0.5, 1.5, N, dtype=torch.float64)
                        (G,) = torch.autograd.grad(ref, x, gg)
                        gg = gg.numpy()
                    else:
                        gg = 0.6
                        (G,) = torch.autograd.grad(ref, x, torch.tensor(gg, dtype=torch.float64))
                    loss, dh, dw = orc.linear_ce(h, w, t, 0.1, reduce_loss=red, g=gg, smoothing=smoothing)
                    what = f"linear {dtype} {N}x{D}x{V} {smoothing} {red}"
                    got = loss if red == "none" else orc.reduce(loss, red, int((t != -100).sum()))
                    _close(got, ref.detach().numpy(), 1e-12, 1e-14, what + " loss")
                    _close(dh, (G @ w.double()).numpy(), 1e-11, 1e-15, what + " dh")
                    _close(dw, (G.T @ h.double()).numpy(), 1e-11, 1e-15, what + " dW")


def pin_linear_finite_differences(orc):
    """dh and dW are the derivatives of the loss (logits kept in FP64 here, so
    the loss is differentiable); 2^-10 steps on a 2^-10 grid are exact."""
    hstep = 2.0 ** -10
    for red in ("none", "mean", "sum"):
        g = torch.Generator().manual_seed(81)
        h = (torch.randint(-1024, 1024, (3, 4), generator=g).double() * hstep).float()
        w = (torch.randint(-1024, 1024, (5, 4), generator=g).double() * hstep).float()
        t = torch.tensor([1, -100, 4])
        gr = np.array([0.7, -1.3, 2.0])
        gs = 1.7

        def objective(hh, ww):
            loss, _, _ = orc.linear_ce(hh, ww, t, 0.2, smoothing="others", round_logits=False,
                                       want_dh=False, want_dw=False)
            return float(np.dot(gr, loss)) if red == "none" else gs * orc.reduce(loss, red, 2)

        _, dh, dw = orc.linear_ce(h, w, t, 0.2, reduce_loss=red, g=gr if red == "none" else gs,
                                  smoothing="others", round_logits=False)
        fd_h = np.zeros_like(dh)
        for i in range(3):
            for d in range(4):
                hp, hm = h.clone(), h.clone()
                hp[i, d] += hstep
                hm[i, d] -= hstep
                fd_h[i, d] = (objective(hp, w) - objective(hm, w)) / (2 * hstep)
        fd_w = np.zeros_like(dw)
        for j in range(5):
            for d in range(4):
                wp, wm = w.clone(), w.clone()
                wp[j, d] += hstep
                wm[j, d] -= hstep
                fd_w[j, d] = (objective(h, wp) - objective(h, wm)) / (2 * hstep)
        _close(dh, fd_h, 1e-4, 1e-7, f"linear finite differences dh {red}")
        _close(dw, fd_w, 1e-4, 1e-7, f"linear finite differences dW {red}")


ALL_PINS = [
    pin_brute_force,
    pin_closed_form_uniform,
    pin_golden_p4_worked_lse,
    pin_golden_p4_other_class_share,
    pin_torch_cross_entropy,
    pin_mean_all_ignored_is_nan,
    pin_finite_differences,
    pin_shift_invariance,
    pin_grad_rows_sum_to_zero,
    pin_sharded_equals_unsharded,
    pin_count_and_rows,
    pin_masked_logits,
    pin_linear_identity_head,
    pin_linear_torch,
    pin_linear_finite_differences,
]

"""ce_shards_fwd_bwd_fused: the vocabulary-shard flow in one launch, each shard
read once, on the GPU through the C ABI, against the FP64 oracle's full-row
loss and gradient (each shard's gradient is that gradient's columns).

Shards as column views of one tensor (in place, disjoint columns) and as
separate buffers; even and ceil-uneven widths (hyper-parallel #269 section
3.1), one shard, tiny shards, shards cut into several chunks; contiguous and
transposed (SQ, B) views; every reduction, both smoothing conventions, masked
(-inf) columns; and workload 4's shape against the three-call shard flow.
"""
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import assert_grad, assert_loss, ignored_rows, orc, raw_bits, rows_f64, say, to_device_view

pytestmark = pytest.mark.gpu


def _g_dev(g, reduce, N):
    if g is None:
        return None
    if reduce == "none":
        return torch.as_tensor(np.asarray(g, np.float32)).cuda()
    return torch.tensor([float(g)], dtype=torch.float32, device="cuda")


def check_shards(x, t, bounds, alpha, reduce, g=None, smoothing="all", separate=False, what=""):
    N = t.numel()
    say(f"[shards fused] {what} {tuple(x.shape)} {x.dtype} S={len(bounds)} a={alpha} {reduce} {smoothing} "
        f"{'buffers' if separate else 'views'}")
    xd, td = to_device_view(x), to_device_view(t)
    if separate:
        shards = [xd[..., a:b].contiguous() for a, b in bounds]
    else:
        shards = [xd[..., a:b] for a, b in bounds]
    loss, n = vce.ce_shards_fwd_bwd_fused(shards, td, alpha, reduce, grad_out=_g_dev(g, reduce, N),
                                          smoothing=smoothing)
    torch.cuda.synchronize()
    o = orc()
    n_ref = o.count_valid(t)
    assert int(n.item()) == n_ref
    ref_rows, _ = o.loss_rows(x, t, alpha, smoothing=smoothing)
    if reduce == "none":
        got = loss.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_rows)
        assert np.array_equal(np.isposinf(got), np.isposinf(ref_rows))
        assert_loss(got[fin], ref_rows[fin], what + " loss rows")
    else:
        ref = o.reduce(ref_rows, reduce, n_ref)
        if reduce == "mean" and n_ref == 0:
            assert math.isnan(loss.item())
        elif math.isinf(ref):
            assert loss.item() == ref
        else:
            assert_loss([loss.item()], [ref], f"{what} {reduce}")
    ref_g = o.grad_rows(x, t, alpha, reduce_loss=reduce, g=g, smoothing=smoothing)
    if separate:
        got_g = np.concatenate([rows_f64(s) for s in shards], axis=1)
    else:
        got_g = rows_f64(xd)
    assert_grad(got_g, ref_g, x.dtype, what + " grad")
    ign = ignored_rows(t)
    if len(ign) and not separate:
        assert not raw_bits(xd, ign).any(), "ignored rows must be +0.0 in every shard"
    return loss


def _logits(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * 2).to(dtype)


LAYOUTS = [(V, S) for V, S in ((5003, 4), (1001, 7), (65, 3), (128000, 16), (400000, 2), (4096, 1))]


@pytest.mark.parametrize("V,S", LAYOUTS, ids=[f"V{v}-S{s}" for v, s in LAYOUTS])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_shard_layouts(V, S, dtype):
    x = _logits((2, 6, V), dtype, seed=V + S)
    t = workloads.random_targets((2, 6), V, seed=V, ignore_frac=0.2)
    bounds = workloads.shard_bounds(V, S)
    check_shards(x, t, bounds, 0.1, "mean", g=0.9, what=f"V={V} S={S}")
    check_shards(x, t, bounds, 0.1, "none", g=np.linspace(-1.0, 2.0, 12), separate=True, what=f"V={V} S={S}")


OPTS = [(red, sm, a) for red in ("none", "mean", "sum") for sm in ("all", "others") for a in (0.0, 0.2)]


@pytest.mark.parametrize("reduce,smoothing,alpha", OPTS, ids=[f"{o[0]}-{o[1]}-a{o[2]}" for o in OPTS])
def test_shard_options_transposed(reduce, smoothing, alpha):
    """The (SQ, B) transposed view of (B, SQ) storage, cut into 5 uneven shards."""
    phys = _logits((3, 8, 9001), torch.bfloat16, seed=31)
    x = phys.transpose(0, 1)
    tp = workloads.random_targets((3, 8), 9001, seed=31, ignore_frac=0.25)
    t = tp.transpose(0, 1)
    g = np.linspace(0.5, 1.5, 24) if reduce == "none" else 0.7
    check_shards(x, t, workloads.shard_bounds(9001, 5), alpha, reduce, g=g, smoothing=smoothing, what="transposed")


@pytest.mark.parametrize("alpha", [0.0, 0.1])
def test_shard_masked_padding(alpha):
    """A vocabulary padded with masked columns at its end (the last shard)."""
    V = 32768 + 128
    x = _logits((2, 8, V), torch.bfloat16, seed=41)
    x[..., 32768:] = -float("inf")
    t = workloads.random_targets((2, 8), 32768, seed=41, ignore_frac=0.1)
    check_shards(x, t, workloads.shard_bounds(V, 4), alpha, "mean", what="masked padding")


def test_shard_rejections():
    x = torch.zeros((1, 4, 100), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((1, 4), dtype=torch.int64, device="cuda")
    a, b = x[..., :50], x[..., 50:]
    with pytest.raises(vce.CeArgumentError):  # dtypes differ
        vce.ce_shards_fwd_bwd_fused([a, b.float()], t)
    with pytest.raises(vce.CeArgumentError):  # no shard
        vce.ce_shards_fwd_bwd_fused([], t)
    with pytest.raises(vce.CeArgumentError):  # rows differ
        vce.ce_shards_fwd_bwd_fused([a, torch.zeros((1, 3, 50), dtype=torch.bfloat16, device="cuda")], t[:, :3])
    with pytest.raises(vce.CeArgumentError):  # more than 16 shards
        vce.ce_shards_fwd_bwd_fused([x[..., i * 5:(i + 1) * 5] for i in range(20)], t)


def test_workload4_against_the_three_call_flow():
    """Workload 4's 4 x [512, 16384] shards: the one-launch flow equals the
    stats / combine / backward flow within the bar and matches the oracle."""
    w = workloads.WORKLOADS[4]
    inp = workloads.generate(w)
    x, t = inp.logits, inp.targets
    bounds = workloads.shard_bounds(w.V, w.shards)
    loss = check_shards(x, t, bounds, w.alpha, "none", g=np.ones(w.rows), separate=True, what="workload 4")
    td = to_device_view(t)
    shards = [x[..., a:b].contiguous().cuda() for a, b in bounds]
    stats = torch.empty((len(bounds), w.rows, 4), dtype=torch.float32, device="cuda")
    for s, (a, b) in enumerate(bounds):
        vce.ce_shard_partial_stats(shards[s], td, a, w.V, stats=stats[s])
    loss3, _, _ = vce.ce_shard_combine(stats, td, w.V, w.alpha, False)
    torch.cuda.synchronize()
    l1, l3 = loss.cpu().numpy().astype(np.float64), loss3.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(l1 - l3) <= 1e-4 * np.maximum(1.0, np.abs(l3)))


AUTOGRAD = [(red, gk) for red in ("none", "mean", "sum") for gk in ("one", "any")]


@pytest.mark.parametrize("reduce,gkind", AUTOGRAD, ids=[f"{r}-{g}" for r, g in AUTOGRAD])
def test_sharded_autograd(reduce, gkind):
    """sharded_cross_entropy: the loss and, after backward, each shard's
    gradient (in the shard's own storage) against the oracle's columns.  A
    factor other than 1 rounds a BF16 gradient twice (staged, then scaled):
    2 x 2^-8 |ref| there, as for parallel_cross_entropy."""
    V, S = 9001, 3
    x = _logits((2, 8, V), torch.bfloat16, seed=61)
    t = workloads.random_targets((2, 8), V, seed=61, ignore_frac=0.2)
    bounds = workloads.shard_bounds(V, S)
    N = t.numel()
    rng = np.random.default_rng(61)
    if reduce == "none":
        g_host = (np.ones(N) if gkind == "one" else rng.uniform(0.2, 2.5, N)).astype(np.float32)
        grad_arg = torch.as_tensor(g_host, device="cuda").view(t.shape)
        g_or = g_host.astype(np.float64)
    else:
        gval = 1.0 if gkind == "one" else 0.3
        grad_arg = torch.tensor(gval, dtype=torch.float32, device="cuda")
        g_or = float(np.float32(gval))
    say(f"[sharded autograd] {reduce} g={gkind}")
    xd, td = to_device_view(x), to_device_view(t)
    shards = [xd[..., a:b].contiguous().requires_grad_(True) for a, b in bounds]
    loss = vce.sharded_cross_entropy(shards, td, 0.1, reduce)
    loss.backward(grad_arg)
    torch.cuda.synchronize()
    o = orc()
    n = o.count_valid(t)
    ref_rows, _ = o.loss_rows(x, t, 0.1)
    if reduce == "none":
        assert tuple(loss.shape) == tuple(t.shape)
        assert_loss(loss.detach().reshape(-1).cpu().numpy(), ref_rows, "sharded autograd rows")
    else:
        assert_loss([float(loss.item())], [o.reduce(ref_rows, reduce, n)], f"sharded autograd {reduce}")
    for sh in shards:
        assert sh.grad is not None and sh.grad.data_ptr() == sh.data_ptr()
    got = np.concatenate([rows_f64(sh.grad) for sh in shards], axis=1)
    ref = o.grad_rows(x, t, 0.1, reduce_loss=reduce, g=g_or, n_valid=n)
    assert_grad(got, ref, torch.bfloat16, "sharded autograd grad", extra_rtol=0.0 if gkind == "one" else 2.0 ** -8)


@pytest.mark.parametrize("reduce", ["none", "mean", "sum"])
def test_shards_no_rows(reduce):
    """No rows: n = 0; the mean is 0/0 = NaN, the sum 0, per-row losses empty."""
    say(f"[shards fused] no rows {reduce}")
    x = torch.zeros((0, 4, 300), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((0, 4), dtype=torch.int64, device="cuda")
    shards = [x[..., a:b] for a, b in workloads.shard_bounds(300, 3)]
    loss, n = vce.ce_shards_fwd_bwd_fused(shards, t, 0.1, reduce)
    torch.cuda.synchronize()
    assert int(n.item()) == 0
    if reduce == "none":
        assert loss.numel() == 0
    elif reduce == "mean":
        assert math.isnan(loss.item())
    else:
        assert loss.item() == 0.0


@pytest.mark.parametrize("reduce", [False, True])
def test_shards_graph_replays(reduce):
    """The shard call captured in a HIP graph: each replay (shards restored in
    between, an eager call on the same workspace interleaved) takes a fresh
    tag from the workspace and matches the eager call bit for bit."""
    V, S = 20000, 3  # shards of 6667 columns: 834 vectors each, whole in one chunk
    x = _logits((2, 9, V), torch.bfloat16, seed=71)
    t = workloads.random_targets((2, 9), V, seed=71, ignore_frac=0.2)
    xd, td = to_device_view(x), to_device_view(t)
    bounds = workloads.shard_bounds(V, S)
    shards = [xd[..., a:b].contiguous() for a, b in bounds]
    pristine = [sh.clone() for sh in shards]
    ws = vce.ce_workspace_init(torch.empty(vce.ce_shards_workspace_bytes(shards, 0.1, reduce), dtype=torch.uint8,
                                           device="cuda"))
    loss = torch.empty(1 if reduce else 18, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")

    def call():
        vce.ce_shards_fwd_bwd_fused(shards, td, 0.1, reduce, loss=loss, n_valid=n, ws=ws)

    def restore():
        for sh, p in zip(shards, pristine):
            sh.copy_(p)

    say(f"[shards graph] eager reference reduce={reduce}")
    call()
    torch.cuda.synchronize()
    ref_grads, ref_loss = [sh.clone() for sh in shards], loss.clone()
    restore()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"[shards graph] replay {rep}")
        restore()
        loss.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for sh, rg in zip(shards, ref_grads):
            assert torch.equal(sh.view(torch.int16), rg.view(torch.int16)), f"replay {rep}: gradient differs"
        assert torch.equal(loss.view(torch.int32), ref_loss.view(torch.int32)), f"replay {rep}: loss differs"
        if rep == 1:
            restore()
            call()
            torch.cuda.synchronize()
    vce.ce_workspace_check(ws)


SHORT = [(V, S, a, sm) for V, S, a, sm in ((3, 3, 1.0, "others"), (17, 13, 0.45, "all"), (64, 16, 0.3, "others"),
                                           (64, 2, 0.0, "all"), (40, 5, 0.8, "all"))]


@pytest.mark.parametrize("V,S,alpha,smoothing", SHORT, ids=[f"V{c[0]}-S{c[1]}-a{c[2]}-{c[3]}" for c in SHORT])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_short_vocabulary_shards(V, S, alpha, smoothing, dtype):
    """A whole vocabulary of at most 64 columns across the shards takes the
    FP64 path (one wave per row gathers its columns from the shards): with few
    columns and heavy smoothing p sits close to a large q, where one FP32
    rounding of p already exceeds the FP32 gradient's absolute floor."""
    g = torch.Generator().manual_seed(V * 31 + S)
    x = (torch.randn((2, 42, V), generator=g) * 6).to(dtype)
    t = workloads.random_targets((2, 42), V, seed=V + S, ignore_frac=0.1)
    bounds = workloads.shard_bounds(V, S) if V % S else [(i * (V // S), (i + 1) * (V // S)) for i in range(S)]
    gr = np.random.default_rng(V).uniform(-2.0, 2.0, 84).astype(np.float32).astype(np.float64)
    for reduce, gg in (("none", gr), ("mean", 1.3), ("sum", None)):
        check_shards(x, t, bounds, alpha, reduce, g=gg, smoothing=smoothing, separate=reduce == "none",
                     what=f"short V={V} S={len(bounds)}")


def test_shards_with_different_layouts():
    """Each shard keeps its own strides: one a column range of a transposed
    (SQ, B) view, one a contiguous buffer, one rows padded inside a wider
    buffer starting off a 16-byte boundary; gradients match the oracle's columns."""
    V = 7001
    bounds = [(0, 2500), (2500, 5000), (5000, V)]
    phys = _logits((3, 6, V), torch.bfloat16, seed=111)          # (B, SQ, V) storage
    x = phys.transpose(0, 1)                                       # the (SQ, B, V) logical view
    tp = workloads.random_targets((3, 6), V, seed=111, ignore_frac=0.2)
    t = tp.transpose(0, 1)
    say("[shards fused] mixed shard layouts")
    xd_t = to_device_view(x)
    s0 = xd_t[..., bounds[0][0]:bounds[0][1]]                      # strided view of the transposed tensor
    s1 = x[..., bounds[1][0]:bounds[1][1]].contiguous().cuda()     # its own contiguous buffer
    w2 = bounds[2][1] - bounds[2][0]
    pad = torch.zeros((6, 3, w2 + 37), dtype=torch.bfloat16)
    pad[..., 3:3 + w2] = x[..., bounds[2][0]:bounds[2][1]]
    s2 = pad.cuda()[..., 3:3 + w2]                                 # padded rows, odd column offset
    td = to_device_view(t)
    loss, n = vce.ce_shards_fwd_bwd_fused([s0, s1, s2], td, 0.1, "none",
                                          grad_out=torch.linspace(0.5, 1.5, 18, device="cuda"))
    torch.cuda.synchronize()
    o = orc()
    assert int(n.item()) == o.count_valid(t)
    ref_rows, _ = o.loss_rows(x, t, 0.1)
    assert_loss(loss.cpu().numpy().astype(np.float64), ref_rows, "mixed layouts loss")
    ref = o.grad_rows(x, t, 0.1, g=np.linspace(0.5, 1.5, 18, dtype=np.float32).astype(np.float64))
    got = np.concatenate([rows_f64(s0), rows_f64(s1), rows_f64(s2)], axis=1)
    assert_grad(got, ref, torch.bfloat16, "mixed layouts grad")

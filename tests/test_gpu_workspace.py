"""The fused call's workspace on the GPU, through the C ABI.

ce_fwd_bwd_fused tags every word its workgroups exchange with a fresh
per-call value, so one workspace prepared once by ce_workspace_init serves
any sequence of calls with no clearing in between; a workspace that was never
prepared (or prepared smaller) makes the call fail loudly: NaN loss and
gradient, n = -1, and CE_EWORKSPACE from ce_workspace_check.  The row count n that
the mean divides by is counted inside the fused kernel, over up to 16 target
slices of at least 2048 rows.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import assert_grad, assert_loss, ignored_rows, orc, rows_f64, say, to_device_view
from test_gpu_parity import check_fused

pytestmark = pytest.mark.gpu


def _logits(shape, dtype, seed, sigma=2.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(dtype)


def _raw_fused(xd, td, alpha, reduce, ws, split_chunks=0):
    """ce_fwd_bwd_fused through the C ABI, without the binding's preparation of ``ws``."""
    N = xd.shape[0] * xd.shape[1]
    loss = torch.empty(1 if reduce else N, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    p = vce.params(alpha, reduce, -100, split_chunks)
    rc = vce.lib.ce_fwd_bwd_fused(ctypes.byref(vce.logits_desc(xd)), ctypes.byref(vce.targets_desc(td)),
                                  ctypes.byref(p), None, ctypes.c_void_p(loss.data_ptr()),
                                  ctypes.c_void_p(n.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, vce.lib.ce_last_error()
    torch.cuda.synchronize()
    return loss, n


def _expect_unprepared(ws):
    with pytest.raises(vce.CeArgumentError) as e:
        vce.ce_workspace_check(ws)
    assert e.value.status == vce._abi.CE_EWORKSPACE
    vce.ce_workspace_check(ws)  # the record was cleared


def test_unprepared_workspace_fails_loudly():
    x = _logits((2, 8, 4096), torch.bfloat16, seed=7)
    t = workloads.random_targets((2, 8), 4096, seed=7, ignore_frac=0.25)
    keep = np.setdiff1d(np.arange(16), ignored_rows(t))
    nb = vce.ce_workspace_bytes(x.cuda(), 0.1, True, split_chunks=2)

    say("[ws] garbage workspace, never prepared")
    ws = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = _raw_fused(xd, td, 0.1, True, ws, split_chunks=2)
    assert math.isnan(loss.item())
    assert int(n.item()) == -1  # the counts travel through the workspace too: not to be trusted there
    assert np.isnan(rows_f64(xd, keep)).all()
    _expect_unprepared(ws)

    say("[ws] workspace prepared smaller than the call needs")
    vce.ce_workspace_init(ws[: nb - 256])
    xd = to_device_view(x)
    loss, _ = _raw_fused(xd, td, 0.1, True, ws, split_chunks=2)
    assert math.isnan(loss.item())
    _expect_unprepared(ws)

    say("[ws] prepared: results match the oracle")
    vce.ce_workspace_init(ws)
    check_fused(x, t, 0.1, True, split_chunks=2, ws=ws, what="prepared")
    vce.ce_workspace_check(ws)


def test_one_workspace_serves_a_sequence_of_calls():
    cases = [((2, 9, 4096), torch.bfloat16, 2, True, 0.1),
             ((3, 5, 8192), torch.float32, 4, False, 0.0),
             ((2, 9, 4096), torch.bfloat16, 2, True, 0.1),  # same shape again: last call's words are stale
             ((1, 40, 1000), torch.bfloat16, 0, True, 0.0),
             ((4, 4, 32003), torch.bfloat16, 3, False, 0.1),
             ((2, 9, 4096), torch.bfloat16, 7, True, 0.1)]
    nb = max(vce.ce_workspace_bytes(torch.empty(s, dtype=dt, device="cuda"), a, r, split_chunks=K)
             for s, dt, K, r, a in cases)
    ws = vce.ce_workspace_init(torch.empty(nb, dtype=torch.uint8, device="cuda"))
    for i, (shape, dtype, K, reduce, alpha) in enumerate(cases):
        x = _logits(shape, dtype, seed=100 + i)
        t = workloads.random_targets(shape[:2], shape[2], seed=100 + i, ignore_frac=0.2)
        check_fused(x, t, alpha, reduce, g=1.0 if reduce else None, split_chunks=K, ws=ws, what=f"sequence {i}")
    vce.ce_workspace_check(ws)


# rows around one slice (2048), several slices, and the 16-slice cap (slices grow past 2048 rows)
@pytest.mark.parametrize("N", [1, 2047, 2049, 6000, 40000])
@pytest.mark.parametrize("reduce", [False, True])
def test_count_over_target_slices(N, reduce):
    # physical (d1, d0) targets passed as the transposed (d0, d1) view: strided count
    d0 = 8 if N % 8 == 0 else 1
    d1 = N // d0
    V = 64
    phys = _logits((d1, d0, V), torch.bfloat16, seed=N)
    x = phys.transpose(0, 1)
    tp = workloads.random_targets((d1, d0), V, seed=N, ignore_frac=0.3)
    t = tp.transpose(0, 1)
    check_fused(x, t, 0.1, reduce, g=1.0 if reduce else None, what=f"count N={d0 * d1}")


@pytest.mark.parametrize("reduce", [False, True])
def test_graph_replays_get_fresh_tags(reduce):
    """A captured fused call replays with the kernel arguments frozen at
    capture; the call's tag comes from the workspace's epoch, advanced by
    every call, so each replay still sees only its own exchanged words.  Each
    replay (the logits restored in between, eager calls on the same
    workspace interleaved) must match an eager call bit for bit."""
    A, B, V, K = 2, 9, 4096, 4  # split rows: the exchange is exercised
    x = _logits((A, B, V), torch.bfloat16, seed=11)
    t = workloads.random_targets((A, B), V, seed=11, ignore_frac=0.2)
    xd, td = to_device_view(x), to_device_view(t)
    pristine = xd.clone()
    nb = vce.ce_workspace_bytes(xd, 0.1, reduce, split_chunks=K)
    ws = vce.ce_workspace_init(torch.empty(nb, dtype=torch.uint8, device="cuda"))
    loss = torch.empty(1 if reduce else A * B, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")

    say(f"[graph] eager reference reduce={reduce}")
    vce.ce_fwd_bwd_fused(xd, td, 0.1, reduce, loss=loss, n_valid=n, ws=ws, split_chunks=K)
    torch.cuda.synchronize()
    ref_grad, ref_loss = xd.clone(), loss.clone()
    check_fused(x, t, 0.1, reduce, g=1.0 if reduce else None, split_chunks=K, what="graph reference")

    say("[graph] capture")
    xd.copy_(pristine)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            vce.ce_fwd_bwd_fused(xd, td, 0.1, reduce, loss=loss, n_valid=n, ws=ws, split_chunks=K)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"[graph] replay {rep}")
        xd.copy_(pristine)
        loss.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(xd.view(torch.int16), ref_grad.view(torch.int16)), f"replay {rep}: gradient differs"
        assert torch.equal(loss.view(torch.int32), ref_loss.view(torch.int32)), f"replay {rep}: loss differs"
        if rep == 1:  # an eager call on the same workspace between replays
            xd.copy_(pristine)
            vce.ce_fwd_bwd_fused(xd, td, 0.1, reduce, loss=loss, n_valid=n, ws=ws, split_chunks=K)
            torch.cuda.synchronize()
            assert torch.equal(xd.view(torch.int16), ref_grad.view(torch.int16))
    vce.ce_workspace_check(ws)


def test_shard_call_with_unprepared_workspace_fails_loudly():
    """The one-launch shard call reads the same workspace record: never
    prepared, its loss and every shard's gradient are NaN and
    ce_workspace_check reports CE_EWORKSPACE; prepared, it matches the oracle."""
    V = 9001
    x = _logits((2, 8, V), torch.bfloat16, seed=17)
    t = workloads.random_targets((2, 8), V, seed=17, ignore_frac=0.25)
    keep = np.setdiff1d(np.arange(16), ignored_rows(t))
    bounds = workloads.shard_bounds(V, 3)
    xd, td = to_device_view(x), to_device_view(t)
    shards = [xd[..., a:b] for a, b in bounds]
    nb = vce.ce_shards_workspace_bytes(shards, 0.1, True)
    say("[ws] shard call, garbage workspace, never prepared")
    ws = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    p = vce.params(0.1, True)
    rc = vce.lib.ce_shards_fwd_bwd_fused(vce._shard_descs(shards), len(shards), ctypes.byref(vce.targets_desc(td)),
                                         ctypes.byref(p), None, ctypes.c_void_p(loss.data_ptr()),
                                         ctypes.c_void_p(n.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, vce.lib.ce_last_error()
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and int(n.item()) == -1
    assert np.isnan(rows_f64(xd, keep)).all()
    _expect_unprepared(ws)

    say("[ws] shard call, prepared: results match the oracle")
    vce.ce_workspace_init(ws)
    xd = to_device_view(x)
    shards = [xd[..., a:b] for a, b in bounds]
    loss, n = vce.ce_shards_fwd_bwd_fused(shards, td, 0.1, True, ws=ws)
    torch.cuda.synchronize()
    o = orc()
    ref_rows, _ = o.loss_rows(x, t, 0.1)
    assert abs(loss.item() - o.mean_loss(ref_rows, o.count_valid(t))) <= 1e-4 * max(1.0, abs(loss.item()))
    vce.ce_workspace_check(ws)


def test_fused_and_shard_calls_share_one_workspace():
    """Fused and shard calls of different shapes and reductions interleaved on
    one workspace prepared once: each matches the same call on a fresh
    workspace bit for bit (the epoch tags keep their exchanged words apart)."""
    cases = [("fused", (2, 9, 40000), 0, True), ("shards", (2, 8, 9001), 3, False), ("fused", (3, 5, 8192), 0, False),
             ("shards", (1, 12, 130000), 5, True), ("fused", (2, 9, 40000), 0, True)]
    need = 0
    for kind, shape, S, red in cases:
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        if kind == "fused":
            need = max(need, vce.ce_workspace_bytes(x, 0.1, red))
        else:
            need = max(need, vce.ce_shards_workspace_bytes(
                [x[..., a:b] for a, b in workloads.shard_bounds(shape[2], S)], 0.1, red))
    shared = vce.ce_workspace_init(torch.empty(need, dtype=torch.uint8, device="cuda"))
    for i, (kind, shape, S, red) in enumerate(cases):
        say(f"[ws] shared workspace, call {i}: {kind} {shape} S={S} reduce={red}")
        x = _logits(shape, torch.bfloat16, seed=100 + i)
        t = workloads.random_targets(shape[:2], shape[2], seed=100 + i, ignore_frac=0.2)
        outs = []
        for ws in (shared, None):
            xd, td = to_device_view(x), to_device_view(t)
            if kind == "fused":
                loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.1, red, ws=ws)
            else:
                loss, n = vce.ce_shards_fwd_bwd_fused([xd[..., a:b] for a, b in workloads.shard_bounds(shape[2], S)],
                                                      td, 0.1, red, ws=ws)
            torch.cuda.synchronize()
            outs.append((xd.view(torch.int16).clone(), loss.view(torch.int32).clone(), int(n.item())))
        assert torch.equal(outs[0][0], outs[1][0]), f"call {i}: gradient differs"
        assert torch.equal(outs[0][1], outs[1][1]), f"call {i}: loss differs"
        assert outs[0][2] == outs[1][2] == orc().count_valid(t)
    vce.ce_workspace_check(shared)


def test_withheld_exchange_words_give_up_with_nan_and_edeadlock():
    """The CE_EDEADLOCK contract, forced from the host with no hang: a test
    hook in the workspace header (word 4, which the library never sets and
    ce_workspace_init zeroes) makes chunk 2 of split row 3 leave its exchange
    words unpublished.  Every chunk of the row reads all of the row's words,
    its own included, so all three chunks' bounded waits give up and every
    workgroup exits: row 3's loss and gradient come out NaN, all other rows
    match the oracle, and ce_workspace_check reports CE_EDEADLOCK once; the
    next call on the same workspace, hook cleared, is exact again."""
    V, K, row, chunk = 12288, 3, 3, 2   # aligned BF16 rows: 1536 vectors, 512 per chunk
    x = _logits((2, 4, V), torch.bfloat16, seed=404)
    t = workloads.random_targets((2, 4), V, seed=404)
    o = orc()
    ref_rows, _ = o.loss_rows(x, t, 0.1)
    ref = o.grad_rows(x, t, 0.1)
    xd, td = to_device_view(x), to_device_view(t)
    ws = vce.ce_workspace_init(torch.empty(vce.ce_workspace_bytes(xd, 0.1, False, split_chunks=K),
                                           dtype=torch.uint8, device="cuda"))
    hook = ws[:40].view(torch.int64)[4:5]
    hook.fill_(((row + 1) << 8) | chunk)
    say(f"[workspace] withheld exchange: row {row}, chunk {chunk} of {K}")
    loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.1, False, split_chunks=K, ws=ws)
    torch.cuda.synchronize()
    with pytest.raises(vce.CeError) as err:
        vce.ce_workspace_check(ws)
    assert err.value.status == vce._abi.CE_EDEADLOCK
    vce.ce_workspace_check(ws)  # the record is cleared
    lv = loss.cpu().numpy().astype(np.float64)
    others = [r for r in range(8) if r != row]
    assert np.isnan(lv[row]) and not np.isnan(lv[others]).any()
    assert_loss(lv[others], ref_rows[others], "rows that did not wait")
    g = rows_f64(xd)
    assert_grad(g[others], ref[others], torch.bfloat16, "rows that did not wait")
    assert np.isnan(g[row]).all(), "the chunks that gave up must write NaN"
    # the hook cleared, the same workspace serves an exact call (a fresh tag)
    hook.zero_()
    xd2 = to_device_view(x)
    loss2, _ = vce.ce_fwd_bwd_fused(xd2, td, 0.1, False, split_chunks=K, ws=ws)
    torch.cuda.synchronize()
    vce.ce_workspace_check(ws)
    assert_loss(loss2.cpu().numpy().astype(np.float64), ref_rows, "after the give-up")
    assert_grad(rows_f64(xd2), ref, torch.bfloat16, "after the give-up")

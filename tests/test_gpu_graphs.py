"""The multi-call paths captured in HIP graphs: ce_forward + ce_backward_inplace,
and the three-call shard flow (ce_shard_partial_stats per shard,
ce_shard_combine, ce_backward_inplace per shard).  Each replay, with its
inputs restored in between and an eager run of the same calls interleaved,
must match the eager result bit for bit.  (The one-launch calls have their own
replay tests beside their other tests.)
"""
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import say, to_device_view

pytestmark = pytest.mark.gpu


def _logits(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * 2).to(dtype)


def _replay_matches_eager(run, buffers, outputs, what):
    """run() enqueues the calls on the current stream; buffers are restored
    before every run; outputs are compared bit for bit with the eager run."""
    pristine = [b.clone() for b in buffers]

    def restore():
        for b, p in zip(buffers, pristine):
            b.copy_(p)

    say(f"[graphs] {what}: eager reference")
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    restore()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"[graphs] {what}: replay {rep}")
        restore()
        for o in outputs:  # the separate outputs start as NaN; the in-place buffers were just restored
            if o.dtype.is_floating_point and not any(o is b for b in buffers):
                o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outputs, ref)):
            view = torch.int16 if o.element_size() == 2 else torch.int32
            assert torch.equal(o.view(view), r.view(view)), f"{what}: replay {rep}, output {k} differs"
        if rep == 1:
            restore()
            run()
            torch.cuda.synchronize()


@pytest.mark.parametrize("form", ["lse", "ex"])
@pytest.mark.parametrize("reduce", ["none", "mean"])
def test_forward_backward_graph_replays(reduce, form):
    x = _logits((2, 9, 5003), torch.bfloat16, seed=81)
    t = workloads.random_targets((2, 9), 5003, seed=81, ignore_frac=0.2)
    xd, td = to_device_view(x), to_device_view(t)
    N = 18
    ws = vce.ce_workspace_init(torch.empty(vce.ce_workspace_bytes(xd, 0.1, reduce), dtype=torch.uint8,
                                           device="cuda"))
    loss = torch.empty(1 if reduce != "none" else N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    g = torch.full((1,) if reduce != "none" else (N,), 0.75, dtype=torch.float32, device="cuda")

    aux = torch.empty((N, 2), dtype=torch.float32, device="cuda") if form == "ex" else None

    def run():
        if form == "ex":
            vce.ce_forward_ex(xd, td, 0.1, reduce, loss=loss, lse=lse, lse_aux=aux, n_valid=n, ws=ws)
        else:
            vce.ce_forward(xd, td, 0.1, reduce, loss=loss, lse=lse, n_valid=n, ws=ws)
        vce.ce_backward_inplace_ex(xd, td, lse, aux, 0.1, reduce, grad_out=g, n_valid=n)

    outs = [xd, loss, lse, n] + ([aux] if form == "ex" else [])
    _replay_matches_eager(run, [xd], outs, f"forward + backward {reduce} {form}")


@pytest.mark.parametrize("form", ["lse", "ex"])
@pytest.mark.parametrize("reduce", ["none", "sum"])
def test_three_call_shard_flow_graph_replays(reduce, form):
    V = 9001
    x = _logits((2, 8, V), torch.bfloat16, seed=82)
    t = workloads.random_targets((2, 8), V, seed=82, ignore_frac=0.2)
    td = to_device_view(t)
    bounds = workloads.shard_bounds(V, 4)
    shards = [x[..., a:b].contiguous().cuda() for a, b in bounds]
    N = 16
    stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device="cuda")
    loss = torch.empty(1 if reduce != "none" else N, dtype=torch.float32, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(vce.ce_combine_workspace_bytes(N, reduce), dtype=torch.uint8, device="cuda")
    g = torch.full((1,) if reduce != "none" else (N,), 1.25, dtype=torch.float32, device="cuda")

    aux = torch.empty((N, 2), dtype=torch.float32, device="cuda") if form == "ex" else None

    def run():
        for s, (a, b) in enumerate(bounds):
            vce.ce_shard_partial_stats(shards[s], td, a, V, stats=stats[s])
        if form == "ex":
            vce.ce_shard_combine_ex(stats, td, V, 0.1, reduce, loss=loss, lse=lse, lse_aux=aux, n_valid=n, ws=ws)
        else:
            vce.ce_shard_combine(stats, td, V, 0.1, reduce, loss=loss, lse=lse, n_valid=n, ws=ws)
        for s, (a, b) in enumerate(bounds):
            vce.ce_backward_inplace_ex(shards[s], td, lse, aux, 0.1, reduce, grad_out=g, n_valid=n, vocab_start=a,
                                       vocab_total=V)

    outs = shards + [stats, loss, lse, n] + ([aux] if form == "ex" else [])
    _replay_matches_eager(run, shards, outs, f"three-call shard flow {reduce} {form}")

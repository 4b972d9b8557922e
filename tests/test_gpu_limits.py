"""The fused call at its limits, on the GPU, against the FP64 oracle:

  * the largest vocabulary automatic chunking takes: 64 chunks of 4096
    16-byte vectors, V = 2^21 BF16 or 2^20 FP32 columns; one vector more is
    refused (CE_ELAYOUT), and the forward + backward calls, which stream any
    row length, take it;
  * a million rows (2^20, the in-kernel count over its 16 target slices of
    65536 rows), for short rows (the FP64 path) and whole 96-column rows;
  * two calls in flight at once on two streams, each with its own workspace,
    and two host threads calling the fused and the shard call concurrently;
  * logits with a large common offset (1000 + N(0, 2^2)).
"""
import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
import workloads
from gpu_util import assert_grad, assert_loss, check_split, orc, rows_f64, say, to_device_view
from test_gpu_parity import check_fused

pytestmark = pytest.mark.gpu


def _logits(shape, dtype, seed, sigma=2.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sigma).to(dtype)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 1 << 21), (torch.float32, 1 << 20)])
def test_largest_vocabulary(dtype, V):
    x = _logits((1, 3, V), dtype, seed=5)
    t = torch.tensor([[7, V - 1, -100]])
    check_fused(x, t, 0.1, True, what=f"largest V={V}")
    check_fused(x, t, 0.1, False, g=np.array([1.0, -0.5, 2.0]), what=f"largest V={V} rows")


def test_vocabulary_beyond_the_fused_limit():
    V = (1 << 21) + 8  # 64 chunks cannot hold it
    x = _logits((1, 2, V), torch.bfloat16, seed=6)
    t = torch.tensor([[3, V - 2]])
    xd, td = to_device_view(x), to_device_view(t)
    with pytest.raises(vce.CeArgumentError):
        vce.ce_fwd_bwd_fused(xd, td, 0.1, True)
    say(f"[limits] streaming forward + backward at V={V}")
    # every element, the targets included, at the stated bar through the lse_aux hand-off
    check_split(x, t, 0.1, False, g=np.ones(2), what=f"beyond the fused limit V={V}", legacy=False)


@pytest.mark.parametrize("V", [32, 96])
def test_a_million_rows(V):
    N = 1 << 20
    x = _logits((16, N // 16, V), torch.bfloat16, seed=V)
    t = workloads.random_targets((16, N // 16), V, seed=V, ignore_frac=0.1)
    rng = np.random.default_rng(V)
    sample = np.unique(np.concatenate([[0, N - 1, 65535, 65536], rng.choice(N, 60, replace=False)]))
    say(f"[limits] {N} rows of {V} columns")
    xd, td = to_device_view(x), to_device_view(t)
    loss, n = vce.ce_fwd_bwd_fused(xd, td, 0.1, True)
    torch.cuda.synchronize()
    o = orc()
    n_ref = o.count_valid(t)
    assert int(n.item()) == n_ref
    ref_rows, _ = o.loss_rows(x, t, 0.1)
    assert_loss([loss.item()], [o.mean_loss(ref_rows, n_ref)], "million rows mean")
    ref = o.grad_rows(x, t, 0.1, reduce_loss=True, rows=sample, n_valid=n_ref)
    assert_grad(rows_f64(xd, sample), ref, torch.bfloat16, "million rows sampled grad")


def test_two_streams_at_once():
    """Each stream's calls use their own workspace; results equal the calls made one at a time."""
    xs = [_logits((2, 64, 32003), torch.bfloat16, seed=s) for s in (8, 9)]
    ts = [workloads.random_targets((2, 64), 32003, seed=s, ignore_frac=0.1) for s in (8, 9)]
    refs = []
    for x, t in zip(xs, ts):
        xd, td = to_device_view(x), to_device_view(t)
        loss, _ = vce.ce_fwd_bwd_fused(xd, td, 0.1, True)
        torch.cuda.synchronize()
        refs.append((loss.clone(), xd.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    dev = [(to_device_view(x), to_device_view(t)) for x, t in zip(xs, ts)]
    wss = [vce.ce_workspace_init(torch.empty(vce.ce_workspace_bytes(d[0], 0.1, True), dtype=torch.uint8,
                                             device="cuda")) for d in dev]
    torch.cuda.synchronize()
    say("[limits] two streams")
    outs = []
    for i in range(2):
        streams[i].wait_stream(torch.cuda.current_stream())
    for i in range(2):
        with torch.cuda.stream(streams[i]):
            outs.append(vce.ce_fwd_bwd_fused(dev[i][0], dev[i][1], 0.1, True, ws=wss[i])[0])
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(outs[i], refs[i][0]), f"stream {i}: loss"
        assert torch.equal(dev[i][0].view(torch.int16), refs[i][1].view(torch.int16)), f"stream {i}: gradient"
        vce.ce_workspace_check(wss[i])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_common_offset(dtype):
    """Logits of 1000 + N(0, 2^2): the loss is shift-invariant, the FP32
    arithmetic around it is not (its error grows like ulp(max |x|)); at this
    offset it stays well inside the bar, for whole and split rows."""
    g = torch.Generator().manual_seed(13)
    x = (1000.0 + torch.randn((2, 8, 32003), generator=g) * 2).to(dtype)
    t = workloads.random_targets((2, 8), 32003, seed=13, ignore_frac=0.1)
    check_fused(x, t, 0.1, True, what=f"offset 1000 {dtype}")
    check_fused(x, t, 0.1, False, g=np.ones(16), split_chunks=5, what=f"offset 1000 split {dtype}")


def test_two_host_threads():
    """Two host threads, each with its own stream and workspace, call the fused
    call and the shard call in a loop at the same time (ctypes releases the
    interpreter lock, so the library's host code runs concurrently); every
    result equals the same call made alone."""
    import threading

    xs = [_logits((2, 32, 20011), torch.bfloat16, seed=s) for s in (21, 22)]
    ts = [workloads.random_targets((2, 32), 20011, seed=s, ignore_frac=0.1) for s in (21, 22)]
    refs = []
    for i, (x, t) in enumerate(zip(xs, ts)):
        xd, td = to_device_view(x), to_device_view(t)
        if i == 0:
            loss, _ = vce.ce_fwd_bwd_fused(xd, td, 0.1, True)
        else:
            loss, _ = vce.ce_shards_fwd_bwd_fused([xd[..., a:b] for a, b in workloads.shard_bounds(20011, 3)],
                                                  td, 0.1, True)
        torch.cuda.synchronize()
        refs.append((loss.clone(), xd.view(torch.int16).clone()))
    say("[limits] two host threads")
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            x, t = xs[i], ts[i]
            td = to_device_view(t)
            base = to_device_view(x)
            xd = base.clone()
            nb = (vce.ce_workspace_bytes(xd, 0.1, True) if i == 0 else
                  vce.ce_shards_workspace_bytes([xd[..., a:b] for a, b in workloads.shard_bounds(20011, 3)], 0.1, True))
            ws = vce.ce_workspace_init(torch.empty(nb, dtype=torch.uint8, device="cuda"))
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for _ in range(30):
                    xd.copy_(base)
                    if i == 0:
                        loss, _ = vce.ce_fwd_bwd_fused(xd, td, 0.1, True, ws=ws)
                    else:
                        loss, _ = vce.ce_shards_fwd_bwd_fused(
                            [xd[..., a:b] for a, b in workloads.shard_bounds(20011, 3)], td, 0.1, True, ws=ws)
                    stream.synchronize()
                    if not (torch.equal(loss, refs[i][0]) and torch.equal(xd.view(torch.int16), refs[i][1])):
                        errors.append(f"thread {i}: result differs")
                        return
            vce.ce_workspace_check(ws)
        except Exception as e:  # reported below
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors

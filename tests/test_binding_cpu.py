"""The Python binding's argument marshalling, on the CPU (the library loads;
no call here reaches the GPU)."""
import pytest

import vocab_cross_entropy_amd as vce
from vocab_cross_entropy_amd import _abi


def test_reduction_and_smoothing_codes():
    assert vce.params(reduce_loss=False).reduce_loss == _abi.CE_REDUCE_NONE
    assert vce.params(reduce_loss=True).reduce_loss == _abi.CE_REDUCE_MEAN
    assert vce.params(reduce_loss="none").reduce_loss == _abi.CE_REDUCE_NONE
    assert vce.params(reduce_loss="mean").reduce_loss == _abi.CE_REDUCE_MEAN
    assert vce.params(reduce_loss="sum").reduce_loss == _abi.CE_REDUCE_SUM
    assert vce.params().smoothing == _abi.CE_SMOOTH_ALL
    assert vce.params(smoothing="others").smoothing == _abi.CE_SMOOTH_OTHERS
    p = vce.params(0.1, "sum", -1, 3, "others")
    assert (p.reduce_loss, p.ignore_idx, p.split_chunks, p.smoothing) == (2, -1, 3, 1)
    assert abs(p.label_smoothing - 0.1) < 1e-7
    # one shared block per distinct value
    assert vce.params(0.1, True) is vce.params(0.1, "mean")


@pytest.mark.parametrize("kw", [dict(reduce_loss="avg"), dict(smoothing="uniform"), dict(reduce_loss="Sum")])
def test_unknown_names_rejected(kw):
    with pytest.raises(vce.CeArgumentError):
        vce.params(**kw)


def test_process_group_needs_more_than_one_gpu():
    with pytest.raises(NotImplementedError):
        vce.parallel_cross_entropy(None, None, dist_process_group=object())


def test_no_shards_rejected_before_any_device_work():
    with pytest.raises(vce.CeArgumentError):
        vce.sharded_cross_entropy([], None)
    with pytest.raises(vce.CeArgumentError):
        vce.ce_shards_fwd_bwd_fused([], None)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says so, before any GPU work."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120, cwd=root)
    assert r.returncode == 2 and "one GPU" in r.stderr, (r.returncode, r.stderr)
    assert r.stdout == ""


def test_host_tensors_refused_before_any_launch():
    """A host (CPU) tensor handed to a call would give a kernel a host pointer:
    the binding refuses it, and wrongly typed or sized outputs, before the
    library sees anything."""
    import torch

    x = torch.zeros((2, 3, 16), dtype=torch.bfloat16)
    t = torch.zeros((2, 3), dtype=torch.int64)
    for call in (lambda: vce.ce_fwd_bwd_fused(x, t), lambda: vce.ce_forward(x, t), lambda: vce.ce_forward_ex(x, t),
                 lambda: vce.ce_backward_inplace(x, t, torch.zeros(6)),
                 lambda: vce.ce_backward_inplace_ex(x, t, torch.zeros(6), torch.zeros((6, 2))),
                 lambda: vce.ce_shard_partial_stats(x, t, 0, 16),
                 lambda: vce.ce_shard_combine_ex(torch.zeros((1, 6, 4)), t, 16),
                 lambda: vce.ce_fwd_bwd_fused_noalloc(x, t, loss=torch.zeros(6), n_valid=torch.zeros(1, dtype=torch.int32)),
                 lambda: vce.ce_shards_fwd_bwd_fused([x], t),
                 lambda: vce.ce_scale_grad_inplace(x, torch.ones(6), True),
                 lambda: vce.parallel_cross_entropy(x, t)):
        with pytest.raises(vce.CeArgumentError):
            call()
    with pytest.raises(vce.CeArgumentError):
        vce.ce_linear_cross_entropy(torch.zeros((4, 8)), torch.zeros((16, 8)), torch.zeros(4, dtype=torch.int64))
    with pytest.raises(vce.CeArgumentError):
        vce.ce_workspace_init(torch.zeros(256, dtype=torch.uint8))

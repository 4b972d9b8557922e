"""The FP64 oracle against its pins (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_out_of_range_target_raises(orc):
    import torch
    x = torch.zeros((1, 2, 4))
    for bad in (4, -1, 99):
        t = torch.tensor([[0, bad]])
        with pytest.raises(oracle.OracleError):
            orc.loss_rows(x, t)
        with pytest.raises(oracle.OracleError):
            orc.grad_rows(x, t)


def test_ignore_index_is_a_parameter(orc):
    import torch
    x = torch.randn((1, 3, 6), generator=torch.Generator().manual_seed(3))
    t = torch.tensor([[-1, 2, -1]])
    loss, _ = orc.loss_rows(x, t, ignore_idx=-1)
    assert loss[0] == 0.0 and loss[2] == 0.0 and loss[1] > 0.0
    with pytest.raises(oracle.OracleError):
        orc.loss_rows(x, t)  # -1 is out of range under the default -100


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("reduce", ["none", "mean", "sum"])
def test_blocked_linear_head_equals_the_loops(dtype, reduce):
    """The oracle's blocked head (a float64 matmul for the logits, for heads
    too large for loops) against or_linear_ce on grid-valued inputs, where
    every product and partial sum is exact: loss rows and dW's sampled columns
    agree to rounding, for blocks that split the rows unevenly."""
    g = torch.Generator().manual_seed(7)
    N, D, V = 37, 24, 301
    h = (torch.randint(-4, 5, (N, D), generator=g).double() / 8).to(dtype)
    w = (torch.randint(-8, 9, (V, D), generator=g).double() / 64).to(dtype)
    t = torch.randint(0, V, (N,), generator=g)
    t[::5] = -100
    gv = np.linspace(-1.0, 2.0, N) if reduce == "none" else 0.7
    orc = oracle.default()
    ref_loss, _, ref_dw = orc.linear_ce(h, w, t, 0.1, reduce_loss=reduce, g=gv, want_dh=False)
    cols = [0, 5, 23]
    seen = []
    for block in (1, 8, 64):
        loss, dwc = orc.linear_ce_blocked(h, w, t, 0.1, reduce_loss=reduce, g=gv, dw_cols=cols, block=block,
                                          on_block=lambda rows, G: seen.append(len(rows)))
        assert np.allclose(loss, ref_loss, rtol=1e-13, atol=1e-13)
        assert np.allclose(dwc, ref_dw[:, cols], rtol=1e-12, atol=1e-13)
    assert sum(seen) == 3 * N

"""The FP64 oracle against its pins (CPU only)."""
import pytest

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

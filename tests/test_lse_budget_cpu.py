"""The budget that the separate-backward tests allow an FP32 lse
(gpu_util.lse_budget) against FP32 arithmetic itself: rows summed on the CPU
with every exponential and every addition rounded to FP32, in the kernels'
schedule (256 or 512 lanes, each summing round-robin 16-byte vectors of 4 or 8
columns in sequence, forward, backward or shuffled, then a tree over the
lanes) and in a balanced tree, the lse then rounded once, must land within the
budget of the FP64 value.  The rows include ones where a single logit holds
nearly all of the probability, so that lse sits near 0 and the sum's rounding,
not ulp(lse), sets the error."""
import math

import numpy as np
import pytest

from gpu_util import lse_budget

f32 = np.float32


def _terms(x):
    m = x.max()
    return m, [f32(np.exp(np.float64(v) - np.float64(m))) for v in x]


def _seq(ts, order):
    d = f32(0.0)
    for i in order:
        d = f32(d + ts[i])
    return d


def _lanes(ts, T, E, how, rng):
    V = len(ts)
    lanes = [[] for _ in range(T)]
    for v in range(-(-V // E)):
        lanes[v % T].extend(range(v * E, min(V, (v + 1) * E)))
    sums = []
    for lane in lanes:
        order = lane[::-1] if how == "backward" else (list(rng.permutation(lane)) if how == "shuffled" else lane)
        sums.append(_seq(ts, order))
    return _tree(sums)


def _tree(ts):
    level = list(ts)
    while len(level) > 1:
        nxt = [f32(level[i] + level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def _lse32(m, d):
    return float(f32(np.float64(m) + math.log(float(d))))


def _lse64(x):
    x = x.astype(np.float64)
    m = x.max()
    return m + math.log(np.exp(x - m).sum())


def _rows(rng):
    # the row of three FP32 logits whose two roundings of d put its lse 3.5 ulp off
    yield np.array([-0.35878554, -7.50582504, -3.56308436], dtype=np.float32)
    for V in (2, 3, 4, 6, 17, 64, 300, 2000, 20000):
        for sigma in (0.5, 2.0, 6.0):
            for _ in range(6 if V < 20000 else 1):
                x = (rng.standard_normal(V) * sigma).astype(np.float32)
                yield x
                y = x.copy()  # one dominant logit: lse near 0
                y[rng.integers(V)] = f32(rng.uniform(-1.0, 1.0))
                y[y != y.max()] -= f32(rng.uniform(3.0, 12.0))
                yield y.astype(np.float32)


def test_fp32_sums_stay_within_the_budget():
    rng = np.random.default_rng(4844)
    worst = 0.0
    for x in _rows(rng):
        m, ts = _terms(x)
        ref = _lse64(x)
        budget = float(lse_budget(np.array([ref]), x.size)[0])
        sums = [_lanes(ts, T, E, how, rng) for T in (256, 512) for E in (4, 8)
                for how in ("forward", "backward", "shuffled")]
        for d in sums + [_tree(ts)]:
            err = abs(_lse32(m, d) - ref)
            worst = max(worst, err / budget)
            assert err <= budget, f"V={x.size}: FP32 lse off by {err:.3e}, budget {budget:.3e}"
    assert worst > 0.1  # the rows do exercise the budget


@pytest.mark.parametrize("lse,vocab,want", [(0.3182, 3, 2.0 ** -25 + (2 + 2 + 4) * 2.0 ** -24),
                                            (12.0, 128000, 2.0 ** -20 + (2 + 17 + 23) * 2.0 ** -24),
                                            (-5.0, 1, 2.0 ** -21 + (2 + 0 + 4) * 2.0 ** -24)])
def test_budget_values(lse, vocab, want):
    assert lse_budget(np.array([lse]), vocab)[0] == pytest.approx(want, rel=1e-12)

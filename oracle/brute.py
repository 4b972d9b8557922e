"""Decimal brute force of the unfused cross-entropy chain, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is the three-step computation that the CANN ops-nn fusion page sets out
as the unfused baseline (section "standard approach: three kernels"):
softmax, then log, then the negative log-likelihood of the target --
generalised to a smoothed target distribution q: either q_j = a/V +
(1-a)[j == t] (smoothing over all classes, torch's convention) or q_t = 1 - a,
q_j = a/(V-1) for j != t (over the other classes, the ops-nn page's kernel,
"pitfall 3").
It deliberately does not use the logsumexp identity the fused method relies
on, and it works in 50-digit decimal arithmetic without any max shift, so it
pins the FP64 oracle independently of how that oracle is written.

Values are Python floats (exact binary fractions, converted exactly to
Decimal).  Meant for N <= 8 rows and V <= 16 columns.
"""
from __future__ import annotations

from decimal import Decimal, localcontext


def _softmax(row, ctx):
    e = [ctx.exp(Decimal(v)) for v in row]
    z = sum(e, Decimal(0))
    return [ei / z for ei in e]


def _target_distribution(V, t, a, smoothing):
    if smoothing == "others":
        return [(1 - a) if j == t else a / (V - 1) for j in range(V)]
    return [a / V + ((1 - a) if j == t else 0) for j in range(V)]


def loss_rows(rows, targets, alpha=0.0, ignore_idx=-100, digits=50, smoothing="all"):
    """Per-row cross-entropy loss as Decimal, via softmax -> log -> NLL."""
    out = []
    with localcontext() as ctx:
        ctx.prec = digits
        a = Decimal(alpha)
        for row, t in zip(rows, targets):
            if t == ignore_idx:
                out.append(Decimal(0))
                continue
            V = len(row)
            if not 0 <= t < V:
                raise ValueError("target out of range")
            probs = _softmax(row, ctx)                      # step 1: softmax
            logp = [ctx.ln(p) for p in probs]               # step 2: log
            q = _target_distribution(V, t, a, smoothing)
            # step 3: NLL; a zero weight contributes nothing (0 log 0 = 0)
            out.append(-sum((qj * lj for qj, lj in zip(q, logp) if qj != 0), Decimal(0)))
    return out


def softmax_rows(rows, digits=50):
    """Row softmax as Decimal (used to check that probabilities sum to one)."""
    with localcontext() as ctx:
        ctx.prec = digits
        return [_softmax(r, ctx) for r in rows]

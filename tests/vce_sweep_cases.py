"""Seeded random configurations for the GPU sweep (tests/test_gpu_sweep.py).

Inputs only: logits, targets, options and shard cut points, drawn from
numpy/torch generators seeded by the case number; nothing of the method's
arithmetic.  Sizes stay at most MAX_ELEMS logits per case, so the FP64 oracle
checks every element of every case in well under a second.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads

N_FUSED = 80
N_SHARDS = 48
N_SPLIT = 48       # ce_forward + ce_backward_inplace
N_SHARD_FLOW = 32  # ce_shard_partial_stats per shard, ce_shard_combine, ce_backward_inplace per shard
N_LINEAR = 24      # ce_linear_cross_entropy (grid-valued inputs: see linear_case)
MAX_ELEMS = 1_500_000
MAX_V = 200_000
MAX_CHUNK_VECS = 4096   # one chunk of the fused call holds at most this many 16-byte vectors
MAX_CHUNKS = 64         # chunks per row
SHORT_ROW = 128         # whole rows of at most this many columns take the library's FP64 path
# Seeds from WIDE_FROM on draw logits of sigma up to 20 (lse near 50) and
# smoothing weights up to 1; each sweep also runs N_WIDE of them.
WIDE_FROM = 20000
N_WIDE = 24


def seeds(n: int) -> list[int]:
    """The sweep's seeds for one kind of call: n ordinary ones, then N_WIDE wide ones."""
    return list(range(n)) + list(range(WIDE_FROM, WIDE_FROM + N_WIDE))


def elems_per_vector(dtype) -> int:
    return 8 if dtype == torch.bfloat16 else 4


def _draw_params(rng: np.random.Generator, v_min: int = 1, wide: bool = False) -> dict:
    """The case's options, from the numpy generator only (no tensors)."""
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    V = int(round(math.exp(rng.uniform(math.log(max(v_min, 1)), math.log(MAX_V)))))
    V = max(v_min, min(MAX_V, V))
    rows_cap = max(1, min(96, MAX_ELEMS // V))
    rows = int(rng.integers(1, rows_cap + 1))
    A = int(rng.integers(1, 5))
    A = min(A, rows)
    B = max(1, rows // A)
    kind = str(rng.choice(["contiguous", "padded", "misaligned", "transposed"]))
    pad = int(rng.integers(1, 40)) if kind in ("padded", "misaligned") else 0
    off = int(rng.integers(1, 8)) if kind == "misaligned" else 0
    sigma = float(rng.choice([0.5, 2.0, 6.0, 20.0] if wide else [0.5, 2.0, 6.0]))
    ignore_frac = float(rng.choice([0.0, 0.1, 0.5, 1.0], p=[0.3, 0.45, 0.2, 0.05]))
    if wide:
        alpha = 0.0 if rng.random() < 0.2 else float(np.float32(rng.uniform(0.01, 1.0)))
    else:
        alpha = 0.0 if rng.random() < 0.3 else float(np.float32(rng.uniform(0.01, 0.5)))
    smoothing = "others" if rng.random() < 0.35 else "all"
    if smoothing == "others" and V == 1 and alpha > 0:
        smoothing = "all"
    reduce = str(rng.choice(["none", "mean", "sum"]))
    rows = A * B
    if reduce == "none":
        g = None if rng.random() < 0.3 else rng.uniform(-2.0, 2.0, rows).astype(np.float32).astype(np.float64)
    else:
        g = None if rng.random() < 0.3 else float(np.float32(rng.uniform(-2.0, 2.0)))
    seed = int(rng.integers(0, 2**31 - 1))
    return dict(dtype=dtype, V=V, A=A, B=B, kind=kind, pad=pad, off=off, sigma=sigma, ignore_frac=ignore_frac,
                alpha=alpha, smoothing=smoothing, reduce=reduce, g=g, seed=seed, wide=wide)


def _materialize(c: dict) -> dict:
    """The case's logits and targets, from its torch seed."""
    A, B, V, dtype, kind, pad, off = c["A"], c["B"], c["V"], c["dtype"], c["kind"], c["pad"], c["off"]
    gen = torch.Generator().manual_seed(c["seed"])
    phys = (torch.randn((A, B, V + pad + off), generator=gen) * c["sigma"]).to(dtype)
    x = phys[..., off:off + V]
    t = workloads.random_targets((A, B), V, seed=c["seed"], ignore_frac=c["ignore_frac"])
    if kind == "transposed":
        x, t = x.transpose(0, 1), t.transpose(0, 1)
    what = (f"{'bf16' if dtype == torch.bfloat16 else 'f32'} V={V} rows={A * B} {kind} sigma={c['sigma']} "
            f"ignored={c['ignore_frac']} a={c['alpha']} {c['smoothing']} {c['reduce']} "
            f"g={'1' if c['g'] is None else 'drawn'}")
    return dict(x=x, t=t, alpha=c["alpha"], smoothing=c["smoothing"], reduce=c["reduce"], g=c["g"], dtype=dtype,
                V=V, what=what, wide=c["wide"])


def _draw_common(rng: np.random.Generator, v_min: int = 1, wide: bool = False):
    return _materialize(_draw_params(rng, v_min, wide))


def fused_case(seed: int) -> dict:
    rng = np.random.default_rng(1000 + seed)
    c = _draw_common(rng, wide=seed >= WIDE_FROM)
    nv = c["V"] // elems_per_vector(c["dtype"])
    K = 0
    if c["V"] > SHORT_ROW and rng.random() < 0.35:  # rows of at most SHORT_ROW columns take the FP64 path
        lo = max(1, -(-nv // MAX_CHUNK_VECS))
        hi = min(MAX_CHUNKS, nv)
        if hi >= lo:
            K = int(rng.integers(lo, hi + 1))
    c["K"] = K
    c["what"] += f" K={K}"
    return c


def shard_case(seed: int) -> dict:
    rng = np.random.default_rng(5000 + seed)
    c = _draw_common(rng, v_min=2, wide=seed >= WIDE_FROM)
    V, E = c["V"], elems_per_vector(c["dtype"])
    S = int(rng.integers(1, min(16, V) + 1))
    while True:
        cuts = np.sort(rng.choice(np.arange(1, V), size=S - 1, replace=False)) if S > 1 else np.array([], int)
        edges = [0] + [int(v) for v in cuts] + [V]
        widest = max(b - a for a, b in zip(edges[:-1], edges[1:]))
        kper = max(1, -(-(widest // E) // MAX_CHUNK_VECS))
        if S * kper <= MAX_CHUNKS:
            break
        S = max(1, S // 2)
    c["bounds"] = list(zip(edges[:-1], edges[1:]))
    c["separate"] = bool(rng.random() < 0.5)
    c["what"] += f" S={S} widths={[b - a for a, b in c['bounds']][:6]}{'...' if S > 6 else ''}"
    return c


def wide_short_row_seeds(kind: str, first: int, last: int, v_lo: int, v_hi: int, min_alpha: float) -> list[int]:
    """Seeds in [first, last) whose fused ("fused") or shard ("shards") case has
    FP32 logits, v_lo <= V <= v_hi and smoothing above min_alpha (numpy draws
    only, so scanning thousands of seeds costs no tensors)."""
    base, v_min = {"fused": (1000, 1), "shards": (5000, 2)}[kind]
    out = []
    for seed in range(first, last):
        c = _draw_params(np.random.default_rng(base + seed), v_min=v_min, wide=seed >= WIDE_FROM)
        if c["dtype"] == torch.float32 and v_lo <= c["V"] <= v_hi and c["alpha"] > min_alpha:
            out.append(seed)
    return out


def split_case(seed: int) -> dict:
    return _draw_common(np.random.default_rng(9000 + seed), wide=seed >= WIDE_FROM)


def shard_flow_case(seed: int) -> dict:
    rng = np.random.default_rng(12000 + seed)
    c = _draw_common(rng, v_min=2, wide=seed >= WIDE_FROM)
    V = c["V"]
    S = int(rng.integers(1, min(16, V) + 1))
    cuts = np.sort(rng.choice(np.arange(1, V), size=S - 1, replace=False)) if S > 1 else np.array([], int)
    edges = [0] + [int(v) for v in cuts] + [V]
    c["bounds"] = list(zip(edges[:-1], edges[1:]))
    c["what"] += f" S={S}"
    return c


def linear_case(seed: int) -> dict:
    """Sizes and options of the chunked head; the inputs themselves are the
    linear tests' grid values (h = k/8, W = m/64), whose products are exact in
    FP32 in any order, so the library's logits equal the oracle's."""
    rng = np.random.default_rng(15000 + seed)
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    N = int(rng.integers(1, 97))
    D = int(rng.integers(1, 257))
    V = int(round(math.exp(rng.uniform(0.0, math.log(20000)))))
    chunk = int(rng.choice([0, 1, int(rng.integers(1, N + 1)), N + 5]))
    alpha = 0.0 if rng.random() < 0.3 else float(np.float32(rng.uniform(0.01, 0.5)))
    smoothing = "others" if (rng.random() < 0.35 and not (V == 1 and alpha > 0)) else "all"
    reduce = str(rng.choice(["none", "mean", "sum"]))
    g = (rng.uniform(0.2, 2.0, N).astype(np.float32).astype(np.float64) if reduce == "none"
         else float(np.float32(rng.uniform(0.2, 2.0))))
    ignore_frac = float(rng.choice([0.0, 0.2, 1.0], p=[0.3, 0.6, 0.1]))
    want = str(rng.choice(["both", "dh", "dw"], p=[0.6, 0.2, 0.2]))
    h_pad = int(rng.choice([0, 0, 5]))
    what = (f"{'bf16' if dtype == torch.bfloat16 else 'f32'} N={N} D={D} V={V} chunk={chunk} a={alpha} "
            f"{smoothing} {reduce} ignored={ignore_frac} want={want} pad={h_pad}")
    return dict(dtype=dtype, N=N, D=D, V=V, chunk=chunk, alpha=alpha, smoothing=smoothing, reduce=reduce, g=g,
                ignore_frac=ignore_frac, want_dh=want != "dw", want_dw=want != "dh", h_pad=h_pad,
                seed=int(rng.integers(0, 2**31 - 1)), what=what)

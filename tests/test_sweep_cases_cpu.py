"""The GPU sweep's case generator on the CPU: every case is within the size
bound, its targets are valid or ignored, its options are ones the calls
accept, and its shard cuts tile the vocabulary within the chunk limit."""
import numpy as np
import torch

import vce_sweep_cases as cases


def _check_common(c):
    x, t = c["x"], c["t"]
    d0, d1, V = x.shape
    assert V == c["V"] and tuple(t.shape) == (d0, d1)
    assert d0 * d1 * V <= cases.MAX_ELEMS
    assert x.stride(2) == 1
    tv = t.reshape(-1).numpy()
    assert np.all((tv == -100) | ((tv >= 0) & (tv < V)))
    assert 0.0 <= c["alpha"] <= (1.0 if c["wide"] else 0.5)
    assert not (c["smoothing"] == "others" and V == 1 and c["alpha"] > 0)
    if c["g"] is not None and c["reduce"] == "none":
        assert len(c["g"]) == d0 * d1


def test_fused_cases_valid():
    kinds = set()
    for seed in cases.seeds(cases.N_FUSED):
        c = cases.fused_case(seed)
        _check_common(c)
        kinds.add(c["what"].split()[3])
        nv = c["V"] // cases.elems_per_vector(c["dtype"])
        if c["K"]:
            assert c["V"] > 64 and 1 <= c["K"] <= min(cases.MAX_CHUNKS, nv)
            assert -(-nv // c["K"]) <= cases.MAX_CHUNK_VECS
    assert kinds == {"contiguous", "padded", "misaligned", "transposed"}


def test_shard_cases_valid():
    for seed in cases.seeds(cases.N_SHARDS):
        c = cases.shard_case(seed)
        _check_common(c)
        b = c["bounds"]
        assert b[0][0] == 0 and b[-1][1] == c["V"] and 1 <= len(b) <= 16
        assert all(lo < hi for lo, hi in b) and all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
        E = cases.elems_per_vector(c["dtype"])
        kper = max(1, -(-(max(hi - lo for lo, hi in b) // E) // cases.MAX_CHUNK_VECS))
        assert len(b) * kper <= cases.MAX_CHUNKS


def test_cases_are_reproducible():
    a, b = cases.fused_case(7), cases.fused_case(7)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["t"], b["t"]) and a["what"] == b["what"]


def test_split_and_shard_flow_cases_valid():
    for seed in cases.seeds(cases.N_SPLIT):
        _check_common(cases.split_case(seed))
    for seed in cases.seeds(cases.N_SHARD_FLOW):
        c = cases.shard_flow_case(seed)
        _check_common(c)
        b = c["bounds"]
        assert b[0][0] == 0 and b[-1][1] == c["V"] and all(lo < hi for lo, hi in b) and len(b) <= 16


def test_linear_cases_valid():
    for seed in range(cases.N_LINEAR):
        c = cases.linear_case(seed)
        assert 1 <= c["N"] <= 96 and 1 <= c["D"] <= 256 and 1 <= c["V"] <= 20000 and c["chunk"] >= 0
        assert c["want_dh"] or c["want_dw"]
        assert not (c["smoothing"] == "others" and c["V"] == 1 and c["alpha"] > 0)

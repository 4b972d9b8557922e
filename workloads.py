"""Seeded synthetic inputs for fused cross-entropy (shared by tests, smoke and bench).

This module only draws random numbers and lays them out; it holds none of the
cross-entropy arithmetic, so both the FP64 oracle and the HIP library can be fed
from it without sharing any of the method's code.

The five workloads take the shapes of the benchmark list on the
TransformerEngineNPU issue #29 page (section 5, typical shapes) and the value,
ignore and smoothing mixes stated for them; the pages' own 1500-shape mass
run and Megatron datasets are not available, so these synthetic inputs stand
in for them.

Draw order for workload k (torch CPU generator seeded 1234 + k):
  1. logits: the physical (A, B, V) tensor in row blocks of 512 rows,
     randn in FP32 times sigma, cast to the storage dtype with
     round-to-nearest-even (torch's own cast);
  2. targets: randint(0, V) over the physical (A, B) shape, int64;
  3. ignored rows: randperm(A*B)[:round(p*A*B)] over the flat physical
     target index, set to ignore_idx;
  4. (spike workloads only) one column per row, randint(0, V), whose logit is
     set to the spike value (exactly representable in BF16).
The "swapped" layout generates the physical (B, SQ, V) tensor and hands out
the transposed (SQ, B, V) view of both logits and targets.
"""
from __future__ import annotations

import dataclasses
import math

import torch

IGNORE_IDX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    key: int
    name: str
    phys: tuple            # physical (A, B) of logits/targets
    V: int
    dtype: torch.dtype
    sigma: float
    ignore_frac: float
    alpha: float
    reduce_loss: bool
    swapped: bool = False  # hand out the transpose(0, 1) view
    spike: float | None = None
    shards: int = 1
    calls: str = "fused"   # "fused" | "split" (forward, then backward) | "shard"

    @property
    def rows(self) -> int:
        return self.phys[0] * self.phys[1]

    @property
    def n_ignored(self) -> int:
        return int(round(self.ignore_frac * self.rows))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == torch.float32 else 2

    @property
    def seed(self) -> int:
        return 1234 + self.key

    def scaled(self, phys=None, V=None, name=None) -> "Workload":
        """Same recipe at another size (used for oracle-sized parity cases)."""
        return dataclasses.replace(self, phys=phys or self.phys, V=V or self.V,
                                   name=name or f"{self.name}@{phys or self.phys}x{V or self.V}")

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "shape": list(self.phys) + [self.V],
            "layout": "swapped (SQ,B,V) transposed view" if self.swapped else "contiguous",
            "dtype": "bf16" if self.dtype == torch.bfloat16 else "f32",
            "rows": self.rows,
            "ignored_rows": self.n_ignored,
            "label_smoothing": self.alpha,
            "reduce_loss": self.reduce_loss,
            "vocab_shards": self.shards,
            "sigma": self.sigma,
            "spike": self.spike,
        }


WORKLOADS = {
    1: Workload(1, "b2_sq128_v4096_f32_split", (2, 128), 4096, torch.float32, 2.0, 0.10, 0.0, False,
                calls="split"),
    2: Workload(2, "sq256_b4_v8192_bf16_swapped_ls0.1_mean", (4, 256), 8192, torch.bfloat16, 3.0, 0.05,
                0.1, True, swapped=True),
    3: Workload(3, "b2_sq512_v32000_bf16_spike20", (2, 512), 32000, torch.bfloat16, 4.0, 0.05, 0.0, False,
                spike=20.0),
    4: Workload(4, "b2_sq256_v65536_bf16_4shards_ls0.1", (2, 256), 65536, torch.bfloat16, 2.0, 0.05, 0.1,
                False, shards=4, calls="shard"),
    5: Workload(5, "b4_sq2048_v128000_bf16_ls0.1_mean", (4, 2048), 128000, torch.bfloat16, 2.0, 0.05, 0.1,
                True),
}


@dataclasses.dataclass
class Inputs:
    """Host tensors of one workload instance."""
    logits_phys: torch.Tensor   # physical storage (A, B, V), contiguous
    targets_phys: torch.Tensor  # physical (A, B) int64, contiguous
    swapped: bool

    @property
    def logits(self) -> torch.Tensor:
        """The (d0, d1, V) view the method is called on."""
        return self.logits_phys.transpose(0, 1) if self.swapped else self.logits_phys

    @property
    def targets(self) -> torch.Tensor:
        return self.targets_phys.transpose(0, 1) if self.swapped else self.targets_phys


def generate(w: Workload, block_rows: int = 512, seed: int | None = None) -> Inputs:
    """Draw one instance of workload ``w`` on the CPU (see module docstring)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    A, B = w.phys
    N, V = A * B, w.V
    flat = torch.empty((N, V), dtype=w.dtype)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        blk = torch.randn((r1 - r0, V), generator=g, dtype=torch.float32)
        blk.mul_(w.sigma)
        flat[r0:r1] = blk.to(w.dtype)
        del blk
    tgt = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    k = w.n_ignored
    if k:
        tgt[torch.randperm(N, generator=g)[:k]] = IGNORE_IDX
    if w.spike is not None:
        cols = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
        flat[torch.arange(N), cols] = torch.tensor(w.spike, dtype=w.dtype)
    return Inputs(flat.view(A, B, V), tgt.view(A, B), w.swapped)


def shard_bounds(V: int, shards: int) -> list[tuple[int, int]]:
    """Uneven split into ceil(V / shards) columns per shard, as on the
    hyper-parallel issue #269 page (section 3.1); the last shard may be short."""
    c = math.ceil(V / shards)
    return [(s * c, min(V, (s + 1) * c)) for s in range(shards) if s * c < V]


def grid_logits(shape, dtype, seed: int, lo: int = -64, hi: int = 64, denom: int = 16) -> torch.Tensor:
    """Logits on the grid k/denom, |k| <= 64: exact in BF16 and FP32, so a
    shift by a multiple of 1/denom stays exact (used for shift-invariance)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    k = torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int64)
    return (k.to(torch.float64) / denom).to(dtype)


def random_targets(shape, V: int, seed: int, ignore_frac: float = 0.0) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    t = torch.randint(0, V, shape, generator=g, dtype=torch.int64)
    n = t.numel()
    k = int(round(ignore_frac * n))
    if k:
        t.view(-1)[torch.randperm(n, generator=g)[:k]] = IGNORE_IDX
    return t

"""Seeded synthetic workloads for the attention forward pass.

This module only draws inputs: it holds none of the method's arithmetic, and
both the HIP path's tests/bench and the fp64 oracle receive the very tensors it
returns.  The pages name no dataset or benchmark suite (their evaluation is on
named hardware only), so these synthetic tensors are the whole workload.

Recipe, per configuration: ``torch.Generator('cpu').manual_seed(seed)``, then
``torch.randn(shape, dtype=float32)`` for Q, then K, then V, in that order;
each is multiplied by its standard deviation and rounded to the storage type
(bfloat16 with round-to-nearest-even, or kept as fp32).  ``scale = 1/sqrt(d)``
as an fp32 value.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str            # "bf16" or "f32"
    seed: int
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        # rounded to fp32, the type the C entry points take
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def nominal_flops(self) -> float:
        """4*B*Hq*N^2*d, halved when causal (the throughput convention)."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five configurations of the throughput/parity matrix.  c4's "N(0,2)" is
# read as standard deviation 2 for Q and K: the configuration states that the
# scaled logits then have std ~4, and std(q.k)/sqrt(d) = sigma_q * sigma_k.
CONFIGS = {
    "c1": Workload("c1", 1, 1, 1, 256, 64, False, "f32", 1,
                   note="single-head fp32, no mask"),
    "c2": Workload("c2", 4, 16, 16, 1024, 64, False, "bf16", 2,
                   note="non-causal bf16 MHA"),
    "c3": Workload("c3", 2, 32, 32, 4096, 128, True, "bf16", 3,
                   note="causal bf16 MHA, N=4096 d=128 (throughput headline)"),
    "c4": Workload("c4", 1, 16, 16, 16384, 128, True, "bf16", 4, 2.0, 2.0, 1.0,
                   note="long causal bf16, wide logits (std ~4)"),
    "c5": Workload("c5", 1, 32, 8, 8192, 128, True, "bf16", 5,
                   note="causal bf16 GQA, 4 query heads per K/V head"),
}


# Workloads beyond the five configurations, for the split-KV path: shapes
# whose direct grid leaves the GPU under-filled or unbalanced.
EXTRA = {
    "s1": Workload("s1", 1, 4, 4, 16384, 128, True, "bf16", 6,
                   note="few heads, long causal: 256 workgroups whose work ranges 1:64"),
    "s2": Workload("s2", 1, 2, 2, 8192, 128, False, "bf16", 7,
                   note="two heads, non-causal: 64 workgroups on 256 CUs"),
}


def make_inputs(w: Workload, device: str = "cpu"):
    """Return (q, k, v) for workload ``w``: q [B,Hq,N,d], k/v [B,Hkv,N,d],
    contiguous, in ``w``'s storage type, drawn on the CPU then moved."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.N, w.d), dtype=torch.float32, generator=g) * w.sigma_q
    k = torch.randn((w.B, w.Hkv, w.N, w.d), dtype=torch.float32, generator=g) * w.sigma_k
    v = torch.randn((w.B, w.Hkv, w.N, w.d), dtype=torch.float32, generator=g) * w.sigma_v
    dt = w.torch_dtype
    q, k, v = (t.to(dt).contiguous() for t in (q, k, v))
    if device != "cpu":
        q, k, v = (t.to(device) for t in (q, k, v))
    return q, k, v


def make_grad(w: Workload, device: str = "cpu"):
    """Return an upstream gradient dO [B,Hq,N,d] for workload ``w``: standard
    normal values from a generator seeded with seed + 1000 (independent of
    the inputs), in ``w``'s storage type."""
    g = torch.Generator("cpu").manual_seed(w.seed + 1000)
    do = torch.randn((w.B, w.Hq, w.N, w.d), dtype=torch.float32, generator=g)
    do = do.to(w.torch_dtype).contiguous()
    return do.to(device) if device != "cpu" else do


def as_f64_numpy(t):
    """Exact upcast of a (CPU or device) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()

"""Seeded synthetic workloads for the GQE attention forward pass.

This module only draws random inputs. It holds none of the method's arithmetic,
so both the HIP path (through the Python binding) and the fp64 oracle can take
their inputs from it without sharing any computation.

Shapes follow the layer described on the pages (16 query heads as 8 KV groups of
2 experts, k=1, one always-on shared head; "Grouped Query Experts" explainer,
technical summary, "Experimental results"), plus the long-context, larger-pool
and extreme-context variants used for parity and timing.

Recipe (identical for every config):
  * torch.Generator on the CPU seeded with 1000 + config id;
  * draw order x, Wr, br (biased-router configs only), Wq, Wk, Wv, Wq_sh, Wo, Wo_gqa;
  * each draw is randn in fp32 times its std, then rounded to bf16 with
    round-to-nearest-even (fp32 configs keep the fp32 values);
  * x ~ N(0, 1); every weight ~ N(0, 1/D); the router offsets br ~ N(0, 0.5)
    (0.5 read as the variance) and stay fp32.
All weights use the [out, in] convention, so y = x @ W.T.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Shape:
    B: int
    T: int
    D: int
    G: int
    M: int
    k: int
    d: int
    dtype: str = "bf16"          # "bf16" or "f32": storage type of x, weights, out
    router_bias: bool = False
    shared_kv_group: int = 0
    variant: str = "full"        # merge: "full" or an ablation ("weighted_concat", "hard_concat", "no_shared")

    @property
    def N(self) -> int:
        return self.B * self.T

    @property
    def slots(self) -> int:      # hard slots + weighted slot + shared slot (one fewer for the ablations)
        return self.G * self.k + (2 if self.variant == "full" else 1)

    @property
    def Hq(self) -> int:         # dense GQA query heads over the same expert pool
        return self.G * self.M

    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


CONFIGS = {
    1: Shape(B=1, T=128, D=128, G=2, M=2, k=1, d=32, dtype="f32"),
    2: Shape(B=8, T=2048, D=1024, G=8, M=2, k=1, d=64),
    3: Shape(B=1, T=32768, D=1024, G=8, M=2, k=1, d=64),
    4: Shape(B=2, T=16384, D=2048, G=8, M=4, k=2, d=64, router_bias=True),
    5: Shape(B=1, T=1048576, D=1024, G=8, M=2, k=1, d=64),
}

CONFIG_NAMES = {
    1: "tiny fp32 layer B1 T128 D128 G2 M2 k1 d32",
    2: "main shape B8 T2048 D1024 G8 M2 k1 d64 bf16",
    3: "long context B1 T32768 D1024 G8 M2 k1 d64 bf16",
    4: "larger pool B2 T16384 D2048 G8 M4 k2 d64 bf16 biased router",
    5: "extreme context B1 T1048576 D1024 G8 M2 k1 d64 bf16",
}


def _draw(gen, shape_, std, dtype):
    t = torch.randn(shape_, generator=gen, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_inputs(s: Shape, seed: int) -> dict:
    """Seeded host tensors for one layer. Returns a dict of CPU torch tensors."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    dt = s.torch_dtype()
    wstd = 1.0 / math.sqrt(s.D)
    out = {}
    out["x"] = _draw(gen, (s.N, s.D), 1.0, dt)
    out["Wr"] = _draw(gen, (s.G * s.M, s.D), wstd, dt)
    out["br"] = (_draw(gen, (s.G * s.M,), math.sqrt(0.5), torch.float32)
                 if s.router_bias else None)
    out["Wq"] = _draw(gen, (s.G * s.M * s.d, s.D), wstd, dt)
    out["Wk"] = _draw(gen, (s.G * s.d, s.D), wstd, dt)
    out["Wv"] = _draw(gen, (s.G * s.d, s.D), wstd, dt)
    out["Wq_sh"] = _draw(gen, (s.d, s.D), wstd, dt)
    out["Wo"] = _draw(gen, (s.D, s.slots * s.d), wstd, dt)
    out["Wo_gqa"] = _draw(gen, (s.D, s.Hq * s.d), wstd, dt)
    return out


def make_grad_output(s: Shape, seed: int) -> torch.Tensor:
    """Seeded gradient of the loss with respect to the layer output, [N, D]
    N(0, 1) in the layer's storage type (the backward's synthetic input)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return _draw(gen, (s.N, s.D), 1.0, s.torch_dtype())


def config_inputs(cid: int) -> tuple[Shape, dict]:
    s = CONFIGS[cid]
    return s, make_inputs(s, 1000 + cid)


def to_f64(t) -> np.ndarray | None:
    """Upcast a (bf16 or fp32) CPU tensor to a float64 numpy array (exact)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def sample_rows(s: Shape, n_rows: int, seed: int) -> np.ndarray:
    """Seeded stratified token rows: t=0 and t=T-1 of batch 0, then rows drawn
    one per equal-width stratum of the flattened N range. Sorted, unique."""
    rng = np.random.default_rng(seed)
    rows = {0, s.T - 1}
    n_rest = max(n_rows - 2, 0)
    if n_rest:
        edges = np.linspace(0, s.N, n_rest + 1).astype(np.int64)
        for a, b in zip(edges[:-1], edges[1:]):
            if b > a:
                rows.add(int(rng.integers(a, b)))
    return np.array(sorted(rows), dtype=np.int64)

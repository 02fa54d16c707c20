"""Seeded synthetic workloads for the sequence-parallel region.

This module only draws inputs; it holds none of the region's arithmetic, and
both the HIP path and the CPU oracle consume what it produces.

Shapes and distributions stand in for the pages' benchmark model (MiniMind,
S=2048, B=2, H=768, bf16, TP=2: "MiniMind-tron: SP optimisation", section 4.1)
and for larger TP=8 shards.  The pages use no dataset.

Recipe: each tensor is drawn in fp32 from its own torch generator seeded with
1000*idx + k (k = t for P_t, 100 residual, 101 gamma, 102 beta, 103 dY,
104 the outlier-row permutation), scaled to its standard deviation, then cast
to the activation type (round to nearest even).  P_t ~ N(0, 1/T),
residual ~ N(0, 1), gamma = 1 + N(0, 0.02^2), beta ~ N(0, 0.02^2), dY ~ N(0, 1).
The long-sequence workload scales 1% of token rows (the same rows in every P_t)
by 100 before the cast.  residual and dY are drawn at full [S,B,H] and sliced,
so the shards of one draw tile a T=1 run.  The dropout seed is 1234.
"""
import math
from dataclasses import dataclass, field

import torch

MASK_SEED = 1234


@dataclass(frozen=True)
class Workload:
    name: str
    idx: int            # seed family
    T: int
    S: int
    B: int
    H: int
    dtype: str          # "bf16" | "f32"
    norm: str           # "rms" | "ln"
    eps: float
    p: float
    shards: tuple
    fwd_only: bool = False
    outlier_frac: float = 0.0
    seed: int = MASK_SEED
    desc: str = field(default="", compare=False)

    @property
    def R(self):
        """Token rows per shard."""
        return (self.S // self.T) * self.B

    @property
    def N(self):
        """Elements per shard."""
        return self.R * self.H

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_T2_S256_B1_H64", 1, 2, 256, 1, 64, "f32", "rms", 1e-6, 0.1, (0,),
                 fwd_only=True, desc="tiny forward-only check, fp32"),
        Workload("minimind_T2_S2048_B2_H768", 2, 2, 2048, 2, 768, "bf16", "rms", 1e-6, 0.1, (0, 1),
                 desc="the pages' benchmark shape, RMSNorm"),
        Workload("layernorm_T8_S4096_B1_H4096", 3, 8, 4096, 1, 4096, "bf16", "ln", 1e-5, 0.1, (3,),
                 desc="LayerNorm, TP=8"),
        Workload("large_hidden_T8_S8192_B2_H8192", 4, 8, 8192, 2, 8192, "bf16", "rms", 1e-6, 0.1, (5,),
                 desc="large hidden, RMSNorm, TP=8"),
        Workload("long_seq_T8_S32768_B1_H8192", 5, 8, 32768, 1, 8192, "bf16", "rms", 1e-6, 0.1,
                 tuple(range(8)), outlier_frac=0.01, desc="long sequence with 1% outlier rows"),
    ]
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, device, seed):
    g = _gen(device, seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def outlier_rows(w, device="cpu"):
    """Token-row indices (into the S*B rows of a full tensor) that are scaled."""
    if w.outlier_frac <= 0:
        return None
    k = int(round(w.outlier_frac * w.S * w.B))
    g = _gen(device, 1000 * w.idx + 104)
    return torch.randperm(w.S * w.B, generator=g, device=device)[:k]


def partial(w, t, device="cpu"):
    """P_t: full [S,B,H] tensor in the activation type."""
    x = _randn((w.S, w.B, w.H), math.sqrt(1.0 / w.T), device, 1000 * w.idx + t)
    rows = outlier_rows(w, device)
    if rows is not None:
        x.view(w.S * w.B, w.H)[rows] *= 100.0
    return x.to(w.torch_dtype)


def residual(w, device="cpu"):
    return _randn((w.S, w.B, w.H), 1.0, device, 1000 * w.idx + 100).to(w.torch_dtype)


def grad_y(w, device="cpu"):
    return _randn((w.S, w.B, w.H), 1.0, device, 1000 * w.idx + 103).to(w.torch_dtype)


def gamma(w, device="cpu"):
    return 1.0 + _randn((w.H,), 0.02, device, 1000 * w.idx + 101)


def beta(w, device="cpu"):
    if w.norm != "ln":
        return None
    return _randn((w.H,), 0.02, device, 1000 * w.idx + 102)


def shard(full, w, j):
    """Rows [j*S/T, (j+1)*S/T) of a full [S,B,H] tensor as an (R, H) view."""
    return full.reshape(-1)[j * w.N:(j + 1) * w.N].view(w.R, w.H)

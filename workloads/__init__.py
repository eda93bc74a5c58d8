"""Seeded synthetic inputs for the attention forward and backward passes.

This module is shared by the oracle-side tests and the GPU-side tests and
benchmark.  It only draws random numbers and rounds them to the storage dtype;
it holds none of the attention arithmetic, so the oracle and the HIP path stay
independent of each other.

Recipe (applies to every workload):
  * generator: ``numpy.random.Generator(PCG64(seed))``;
  * draw order: Q, then K, then V, each ``standard_normal(shape,
    dtype=float32)`` in C order, multiplied by ``sigma``; the shape is
    [B, H, S, d] for Q and [B, Hkv, S, d] for K and V (Hkv = H unless the
    workload has grouped key/value heads);
  * rounding: round-to-nearest-even to the storage dtype (torch CPU ``.to``);
  * output gradient for the backward pass (``make_grad``): its own generator
    ``PCG64(seed)`` over [B, H, S, d], ``standard_normal`` float32, rounded
    the same way (callers pass a seed distinct from the inputs' seed);
  * optional outliers: after the three draws, for every (b, h) of K in (b, h)
    order, ``rng.choice(S, floor(0.01 * S), replace=False)`` picks key rows that
    are multiplied by 8 (a power of two, so scaling before or after rounding
    gives identical bits).

The named workloads are the five attention configurations the benchmark and
the parity tests use (tiny fp32, causal d=64, long causal prefill d=128,
sliding-window d=128, non-causal d=256 fp16), the outlier variant of the
causal d=64 case, and the long causal prefill with grouped key/value heads
(32 query heads over 8 key/value heads).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_grad", "generate", "input_digest",
           "TORCH_DTYPES"]

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    d: int
    dtype: str           # "f32" | "f16" | "bf16"
    mask: str            # "none" | "causal" | "window"
    window: int = 0      # keys visible to query i: i - window < j <= i
    sigma: float = 1.0
    seed: int = 0
    outliers: bool = False
    Hkv: int = 0         # key/value heads; 0 means H (plain multi-head attention)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask lets through, per (b, h) x B*H."""
        S = self.S
        if self.mask == "none":
            per = S * S
        elif self.mask == "causal":
            per = S * (S + 1) // 2
        else:
            W = self.window
            if W >= S:
                per = S * (S + 1) // 2
            else:
                # rows i < W see i + 1 keys, the remaining S - W rows see W keys
                per = W * (W + 1) // 2 + (S - W) * W
        return per * self.B * self.H

    def flops(self) -> float:
        """Algorithmic forward FLOPs: 4*d per visible pair (2 for Q.K, 2 for P.V)."""
        return 4.0 * self.d * self.visible_pairs()

    def compulsory_bytes(self) -> int:
        """Q, K, V read once plus O and the fp32 LSE written once."""
        esz = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        n = self.B * self.H * self.S
        nkv = self.B * self.kv_heads * self.S
        return (2 * n + 2 * nkv) * self.d * esz + 4 * n


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 256, 64, "f32", "none", seed=1000),
    "causal_d64": Workload("causal_d64", 2, 8, 1024, 64, "bf16", "causal", seed=1001),
    "causal_d64_outliers": Workload("causal_d64_outliers", 2, 8, 1024, 64, "bf16",
                                    "causal", seed=1001, outliers=True),
    "prefill_8k_d128": Workload("prefill_8k_d128", 1, 32, 8192, 128, "bf16", "causal",
                                seed=1002),
    "window_18k_d128": Workload("window_18k_d128", 1, 16, 18432, 128, "bf16", "window",
                                window=4096, seed=1003),
    "full_d256_f16": Workload("full_d256_f16", 4, 16, 4096, 256, "f16", "none",
                              sigma=0.5, seed=1004),
    "prefill_8k_d128_gqa4": Workload("prefill_8k_d128_gqa4", 1, 32, 8192, 128, "bf16",
                                     "causal", seed=1005, Hkv=8),
}


def make_inputs(B: int, H: int, S: int, d: int, dtype: str, seed: int,
                sigma: float = 1.0, outliers: bool = False, Hkv: int | None = None):
    """Return (q, k, v) as contiguous CPU torch tensors of ``dtype``; k and v
    have ``Hkv`` heads (default H)."""
    Hkv = Hkv or H
    rng = np.random.Generator(np.random.PCG64(seed))
    arrs = []
    for shape in ((B, H, S, d), (B, Hkv, S, d), (B, Hkv, S, d)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        arrs.append(x)
    if outliers:
        n_out = int(math.floor(0.01 * S))
        kx = arrs[1]
        for b in range(B):
            for h in range(Hkv):
                idx = rng.choice(S, n_out, replace=False)
                kx[b, h, idx, :] *= np.float32(8.0)
    tdt = TORCH_DTYPES[dtype]
    return tuple(torch.from_numpy(a).to(tdt).contiguous() for a in arrs)


def make_grad(B: int, H: int, S: int, d: int, dtype: str, seed: int):
    """The gradient of the output, dO: a contiguous CPU tensor [B, H, S, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, H, S, d), dtype=np.float32)
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype]).contiguous()


def generate(w: Workload):
    return make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)


def input_digest(*tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def with_shape(w: Workload, **kw) -> Workload:
    return replace(w, **kw)

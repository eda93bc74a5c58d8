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
           "TORCH_DTYPES", "DecodeWorkload", "DECODE_WORKLOADS", "make_decode_inputs",
           "blocks_needed", "kv_bytes_per_token", "generate_decode"]

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


# ---------------------------------------------------------------------------
# Decoding over a paged key/value cache.
#
# Recipe (``make_decode_inputs``): generator PCG64(seed); draw order
#   1. the context lengths, ``integers(ctx_lo, ctx_hi + 1, size=B)`` (unless
#      the caller passes them);
#   2. Q [B, H, n_q, d], standard normal float32, C order;
#   3. the K cache, then the V cache, each [num_blocks, Hkv, bs, d] standard
#      normal float32 in C order, drawn block by block;
#   4. the placement: ``permutation(num_blocks)``; request b takes the next
#      ceil(n_b / bs) physical blocks of it, in request order, for its logical
#      blocks 0, 1, ... (so a request's blocks are scattered over the pool);
#      table entries past a request's last block are -1.
# num_blocks = sum_b ceil(n_b / bs) + extra_blocks (unowned blocks hold random
# data the kernel must never read).  Values are rounded RNE to the storage
# dtype.


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """Physical blocks a request of n_tokens occupies (the last one partly)."""
    return -(-int(n_tokens) // int(block_size)) if n_tokens > 0 else 0


def kv_bytes_per_token(kv_heads: int, d: int, esz: int, layers: int = 1) -> int:
    """Cache bytes one token occupies: a key and a value row for every
    key/value head (of every layer)."""
    return 2 * layers * kv_heads * d * esz


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int               # concurrent requests
    H: int               # query heads
    Hkv: int             # key/value heads
    n_q: int             # new tokens per request (query rows)
    d: int
    dtype: str           # "f16" | "bf16"
    block_size: int
    ctx_lo: int          # context lengths drawn uniformly from [ctx_lo, ctx_hi]
    ctx_hi: int
    seed: int
    extra_blocks: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_ctx(self) -> int:
        return self.ctx_hi

    @property
    def esz(self) -> int:
        return {"f16": 2, "bf16": 2}[self.dtype]

    def ctx_lens(self) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64(self.seed))
        return rng.integers(self.ctx_lo, self.ctx_hi + 1, size=self.B)

    def visible_pairs(self, ctx) -> int:
        """(query row, cached token) pairs over all heads: row i of a request
        with n tokens sees n - n_q + i + 1 of them."""
        per_req = sum(sum(max(int(n) - self.n_q + i + 1, 0) for i in range(self.n_q))
                      for n in ctx)
        return per_req * self.H

    def flops(self, ctx) -> float:
        return 4.0 * self.d * self.visible_pairs(ctx)

    def compulsory_bytes(self, ctx) -> int:
        """Every cached key and value row of every request read once, the
        queries read and the outputs (plus fp32 LSE) written once; the block
        table and context lengths are negligible and not counted."""
        tokens = int(np.sum(np.asarray(ctx)))
        qo = 2 * self.B * self.H * self.n_q * self.d * self.esz + 4 * self.B * self.H * self.n_q
        return tokens * kv_bytes_per_token(self.Hkv, self.d, self.esz) + qo


DECODE_WORKLOADS = {
    # one layer of an OPT-13B-shaped model (hidden 5120 = 40 heads x 128, fp16,
    # multi-head), 256 concurrent requests with contexts up to its 2,048-token
    # window, 16-token blocks, one new token each
    "decode_opt13b_b256": DecodeWorkload("decode_opt13b_b256", 256, 40, 40, 1, 128, "f16", 16,
                                         1, 2048, seed=1100, extra_blocks=64),
    # grouped heads (32 over 8), few long requests: the context is split over
    # several work-groups and merged
    "decode_gqa_long": DecodeWorkload("decode_gqa_long", 4, 32, 8, 1, 128, "bf16", 16,
                                      16384, 32768, seed=1101, extra_blocks=16),
    # four new tokens per request (causal among themselves)
    "decode_gqa_nq4": DecodeWorkload("decode_gqa_nq4", 32, 32, 8, 4, 128, "bf16", 16,
                                     512, 4096, seed=1102, extra_blocks=16),
    # grouped heads, 8 query heads per key/value head (64 over 8, one new
    # token), 16 requests of 1K-8K tokens
    "decode_gqa8": DecodeWorkload("decode_gqa8", 16, 64, 8, 1, 128, "bf16", 16, 1024, 8192,
                                  seed=1104, extra_blocks=16),
    # grouped heads at serving scale: 256 requests of up to 4K tokens, 32 query
    # heads over 8 key/value heads (about 2 GB of cache per step)
    "decode_gqa_b256": DecodeWorkload("decode_gqa_b256", 256, 32, 8, 1, 128, "bf16", 16, 1,
                                      4096, seed=1105, extra_blocks=64),
    # small case the oracle finishes at once
    "decode_small": DecodeWorkload("decode_small", 3, 4, 2, 2, 64, "bf16", 16, 1, 300,
                                   seed=1103, extra_blocks=5),
}


def _normal_blocks(rng, shape, tdt, chunk_rows=4096):
    """standard_normal float32 over `shape` in C order, drawn in chunks of the
    leading dimension (same values as one draw), rounded to tdt."""
    out = torch.empty(shape, dtype=tdt)
    n = shape[0]
    for lo in range(0, n, chunk_rows):
        hi = min(n, lo + chunk_rows)
        x = rng.standard_normal((hi - lo,) + tuple(shape[1:]), dtype=np.float32)
        out[lo:hi] = torch.from_numpy(x).to(tdt)
    return out


def make_decode_inputs(B: int, H: int, Hkv: int, n_q: int, d: int, dtype: str,
                       block_size: int, seed: int, ctx_lens=None, ctx_range=None,
                       extra_blocks: int = 0, max_blocks: int | None = None):
    """Return (q, k_cache, v_cache, block_table, ctx_lens) as CPU tensors
    (block_table and ctx_lens int32) following the recipe above."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if ctx_lens is None:
        lo, hi = ctx_range
        ctx_lens = rng.integers(lo, hi + 1, size=B)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    tdt = TORCH_DTYPES[dtype]
    q = torch.from_numpy(rng.standard_normal((B, H, n_q, d), dtype=np.float32)).to(tdt)
    need = [blocks_needed(int(n), block_size) for n in ctx]
    num_blocks = sum(need) + extra_blocks
    if num_blocks == 0:
        num_blocks = 1
    k_cache = _normal_blocks(rng, (num_blocks, Hkv, block_size, d), tdt)
    v_cache = _normal_blocks(rng, (num_blocks, Hkv, block_size, d), tdt)
    perm = rng.permutation(num_blocks)
    mb = max(max(need, default=0), 1) if max_blocks is None else max_blocks
    table = np.full((B, mb), -1, dtype=np.int32)
    off = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[off:off + nb]
        off += nb
    return (q.contiguous(), k_cache, v_cache, torch.from_numpy(table),
            torch.from_numpy(ctx.astype(np.int32)))


def generate_decode(w: DecodeWorkload):
    """Inputs of a named decode workload (its context lengths are the first
    draw of the stream, the same values ``w.ctx_lens()`` returns)."""
    return make_decode_inputs(w.B, w.H, w.Hkv, w.n_q, w.d, w.dtype, w.block_size, w.seed,
                              ctx_range=(w.ctx_lo, w.ctx_hi), extra_blocks=w.extra_blocks)

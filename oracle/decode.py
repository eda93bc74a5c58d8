"""Plain fp64 CPU oracle for attention decoding over a paged key/value cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module; it shares no code with the HIP path.

Source: the aicomputerinstitute.com grade-12 chapter on flash attention and
memory-efficient attention variants, sections "A different bottleneck: the KV
cache during inference" and "PagedAttention: memory management borrowed from
an operating system".  During autoregressive decoding each new token attends
over the keys and values of every earlier token, which a serving system keeps
in a cache.  The paged cache cuts that memory into fixed-size physical blocks
placed anywhere in device memory; each request owns a block table that maps
its logical token positions to physical blocks, and the attention kernel
walks the table to gather the blocks it needs.  The attention itself is the
unchanged exact attention (the chapter's section "It's worth being precise
about the boundary" pairs the two: fused exact attention once the blocks are
in hand, block tables for where they live).

What is computed, for request b with context length n_b:
  * token t (0 <= t < n_b) lives in physical block P = block_table[b, t // bs],
    slot t % bs: its key for key/value head g is k_cache[P, g, t % bs, :], and
    likewise its value;
  * a block-table entry outside [0, num_blocks) holds no token: positions it
    would cover are not attended (a padding entry such as -1 is harmless);
  * n_b = ctx_lens[b] clamped to [0, min(max_ctx, max_blocks * bs)];
  * the request's n_q query rows are its newest tokens, at positions
    n_b - n_q + i (i = 0 .. n_q - 1); their keys and values are already in the
    cache, and row i attends to positions t <= n_b - n_q + i (causal; with
    n_q = 1 that is every cached token);
  * query head h uses key/value head h // (H / Hkv);
  * O and LSE are the plain softmax attention of the row over its visible
    keys, as in ``oracle.attention``; a row with no visible key gets O = 0 and
    LSE = -inf.

Shapes: q [B, H, n_q, d]; k_cache, v_cache [num_blocks, Hkv, bs, d];
block_table [B, max_blocks] (integers); ctx_lens [B].  Everything is converted
exactly to fp64 before any arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64, _softmax_rows

__all__ = ["paged_token_slots", "paged_gather", "paged_decode_ref"]


def paged_token_slots(table_row, n_tokens: int, block_size: int, num_blocks: int):
    """Where each logical token of one request lives.

    Returns (positions, blocks, slots): the logical positions t < n_tokens
    whose block-table entry is a valid physical block, with that block and
    the slot t % block_size inside it.
    """
    table_row = np.asarray(table_row).astype(np.int64)
    t = np.arange(max(int(n_tokens), 0), dtype=np.int64)
    logical = t // block_size
    if logical.size and logical[-1] >= table_row.shape[0]:
        raise ValueError("context longer than the block table")
    phys = table_row[logical]
    ok = (phys >= 0) & (phys < num_blocks)
    return t[ok], phys[ok], (t % block_size)[ok]


def paged_gather(cache, table_row, n_tokens: int, kv_head: int):
    """Logical positions and the [n, d] rows of one head of one request."""
    num_blocks, _, bs, _ = cache.shape
    pos, phys, slot = paged_token_slots(table_row, n_tokens, bs, num_blocks)
    if hasattr(cache, "detach"):  # torch: index first, then convert the rows only
        import torch
        rows = cache[torch.from_numpy(phys), kv_head, torch.from_numpy(slot), :]
    else:
        rows = cache[phys, kv_head, slot, :]
    return pos, _as_f64(rows)


def _context_length(ctx, max_ctx, max_blocks, bs):
    n = int(ctx)
    cap = max_blocks * bs
    if max_ctx is not None:
        cap = min(cap, int(max_ctx))
    return min(max(n, 0), cap)


def paged_decode_ref(q, k_cache, v_cache, block_table, ctx_lens, max_ctx=None, scale=None,
                     requests=None):
    """Exact decode attention over a paged cache (see the module docstring).

    Returns (O [B, H, n_q, d], LSE [B, H, n_q]) in fp64.  ``requests``
    optionally restricts the work to a list of request indices (other rows
    are NaN).
    """
    B, H, n_q, d = q.shape
    num_blocks, Hkv, bs, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes disagree with q")
    if H % Hkv != 0:
        raise ValueError("key/value heads must divide query heads")
    table = np.asarray(block_table)
    ctx = np.asarray(ctx_lens)
    if table.shape[0] != B or ctx.shape != (B,):
        raise ValueError("block table / context lengths disagree with the batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = H // Hkv
    o = np.full((B, H, n_q, d), np.nan)
    lse = np.full((B, H, n_q), np.nan)
    for b in (range(B) if requests is None else requests):
        n = _context_length(ctx[b], max_ctx, table.shape[1], bs)
        rows = n - n_q + np.arange(n_q)               # positions of the query rows
        for g in range(Hkv):
            pos, kg = paged_gather(k_cache, table[b], n, g)
            _, vg = paged_gather(v_cache, table[b], n, g)
            vis = pos[None, :] <= rows[:, None]       # [n_q, n_valid]
            for h in range(g * group, (g + 1) * group):
                if kg.shape[0] == 0:                  # nothing cached: empty rows
                    o[b, h], lse[b, h] = 0.0, -np.inf
                    continue
                qh = _as_f64(q[b, h])
                s = scale * (qh @ kg.T)
                s = np.where(vis, s, -np.inf)
                p, m, l = _softmax_rows(s)
                o[b, h] = p @ vg
                with np.errstate(divide="ignore"):
                    lse[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse

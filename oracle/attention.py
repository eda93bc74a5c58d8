"""Plain, slow, fp64 CPU oracle for exact attention with the online softmax.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: it exists so that tests, the package smoke check and the
benchmark's CPU-baseline leg can compare the HIP kernels against an obviously
correct computation.  It shares no code with the HIP path.

What is computed (sources are the three pages on the subject):

* ``attention_ref`` -- the plain definition, materialising the score matrix
  S = scale * Q K^T and the probability matrix P = softmax(S) row by row in
  fp64, then O = P V.  The definition of attention as softmax of scaled
  query-key dot products applied to V is given in "FlashAttention: Why Tiling
  Attention Makes Transformers Fast Without Changing the Result" (Dev.to),
  section "The problem is memory, not arithmetic", and in the aicomputer-
  institute grade-12 chapter on flash attention, section "Two kinds of memory
  live on every GPU".  The max-subtracted (safe) softmax follows the Dev.to
  article's section "Why softmax seems to block tiling".  Every page says the
  tiled method reaches this same result up to rounding order, so the
  definition itself is the oracle.
* ``attention_tiled_ref`` -- the running-statistics procedure (running max m,
  running sum l, unnormalised output accumulator rescaled by exp(m_old -
  m_new), one divide at the end), in the order the aicomputerinstitute chapter
  gives it in "Tiling and the running (online) softmax" and traces in "Worked
  example: tracing the running statistics by hand".  It is used only to pin
  the oracle against itself (one-pass == tiled for every block size).
* the per-row logsumexp emitted next to O is the natural log of the softmax
  denominator over the visible, scaled scores, LSE = m + ln(l).  The
  foundry.adhana.ai page "FlashAttention: IO-aware attention kernels", section
  "In and out", names it as the second output.

Masks (section "The knobs" of the foundry.adhana.ai page names causal and
sliding-window masks as the natively supported kinds):
  none   : every key j is visible to query i;
  causal : j <= i;
  window : i - window < j <= i   (window counts the diagonal; window >= S is
           the causal mask).
A row with no visible key (not reachable through the library, whose masks
always keep the diagonal) gets O = 0 and LSE = -inf; the foundry page's
"Failure modes" section names such rows as the NaN hazard to guard.

Gradients (``attention_bwd_ref``): the Dev.to article's section "The backward
pass: recompute instead of storing" gives dV = P^T dO, dP = dO V^T, dS from
the softmax Jacobian applied to dP, and dQ, dK by the matrix-product rules;
here P is simply materialised, since the oracle is the plain definition.

Grouped key/value heads: the Dev.to article's section "Using it in practice"
says later variants of the method support grouped-query attention without
spelling it out.  The plain reading, taken here, is the usual one: K and V
carry Hkv heads, Hkv divides the H query heads, and query head h attends with
key/value head h // (H / Hkv) (Hkv = H is ordinary multi-head attention,
Hkv = 1 multi-query attention).  Nothing else changes.

Inputs are any real arrays (numpy or torch CPU) of shape [B, H, S, d] (K and V:
[B, Hkv, S, d]); they are converted exactly to fp64 before any arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["visible", "attention_ref", "attention_probs_ref", "attention_tiled_ref",
           "attention_rows_ref", "kv_head", "attention_bwd_rows_ref", "attention_bwd_ref"]

_MASKS = ("none", "causal", "window")


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: go through fp64 exactly
        import torch
        return x.detach().to("cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def visible(rows: np.ndarray, cols: np.ndarray, mask: str, window: int | None) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: key cols[j] visible to query rows[i]."""
    if mask not in _MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    r = np.asarray(rows)[:, None]
    c = np.asarray(cols)[None, :]
    if mask == "none":
        return np.ones((r.shape[0], c.shape[1]), dtype=bool)
    vis = c <= r
    if mask == "window":
        if window is None or window < 1:
            raise ValueError("window mask needs window >= 1")
        vis &= c > r - window
    return vis


def _softmax_rows(scores: np.ndarray):
    """Safe softmax of each row (-inf entries are invisible keys).

    Returns (P, m, l): probabilities, row max, and the max-shifted denominator.
    A row with every entry -inf yields P = 0, m = -inf, l = 0.
    """
    m = scores.max(axis=-1)
    dead = np.isneginf(m)
    shift = np.where(dead, 0.0, m)
    e = np.exp(scores - shift[..., None])          # exp(-inf) = 0
    l = e.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(dead[..., None], 0.0, e / np.where(dead, 1.0, l)[..., None])
    return p, m, l


def attention_probs_ref(q, k, mask="none", window=None, scale=None):
    """Materialise P = softmax(scale * q k^T) for one head.

    q: [Sq, d], k: [Sk, d] (query index i runs over 0..Sq-1, key index over
    0..Sk-1; masks compare the two indices directly).  Returns (P, m, l) in fp64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = scale * (q @ k.T)
    vis = visible(np.arange(q.shape[0]), np.arange(k.shape[0]), mask, window)
    s = np.where(vis, s, -np.inf)
    return _softmax_rows(s)


def attention_rows_ref(q, k, v, rows, mask="none", window=None, scale=None):
    """Exact attention for the query indices ``rows`` of one head.

    q, k, v: [S, d].  Returns (O [len(rows), d], LSE [len(rows)]) in fp64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = scale * (q[rows] @ k.T)
    vis = visible(rows, np.arange(k.shape[0]), mask, window)
    s = np.where(vis, s, -np.inf)
    p, m, l = _softmax_rows(s)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(np.isneginf(m), -np.inf, m + np.log(np.where(l > 0, l, 1.0)))
    return o, lse


def kv_head(h: int, n_heads: int, n_kv_heads: int) -> int:
    """Key/value head that query head h attends with (grouped heads)."""
    if n_kv_heads < 1 or n_heads % n_kv_heads:
        raise ValueError(f"{n_kv_heads} key/value heads do not divide {n_heads} query heads")
    return h // (n_heads // n_kv_heads)


def attention_ref(q, k, v, mask="none", window=None, scale=None, row_chunk=2048,
                  heads=None):
    """Exact fp64 attention over [B, H, S, d] queries and [B, Hkv, S, d] keys
    and values (Hkv divides H; Hkv = H is plain multi-head attention).

    For every (b, h) and every chunk of at most ``row_chunk`` query rows the
    scaled score block and its probabilities are materialised in full, against
    key/value head kv_head(h, H, Hkv).  ``heads`` optionally restricts the work
    to a list of (b, h) pairs (the other heads of the result are left as NaN).
    Returns (O [B,H,S,d], LSE [B,H,S]) in fp64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, S, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, d) or v.shape[:3] != (B, Hkv, S):
        raise ValueError("q, k, v shapes disagree")
    dv = v.shape[-1]
    o = np.full((B, H, S, dv), np.nan)
    lse = np.full((B, H, S), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        g = kv_head(h, H, Hkv)
        for r0 in range(0, S, row_chunk):
            rows = np.arange(r0, min(S, r0 + row_chunk))
            o[b, h, rows], lse[b, h, rows] = attention_rows_ref(
                q[b, h], k[b, g], v[b, g], rows, mask, window, scale)
    return o, lse


def attention_tiled_ref(q, k, v, mask="none", window=None, scale=None, block=64,
                        trace=None):
    """Running-statistics (online softmax) evaluation over key blocks, fp64.

    q, k, v: [S, d] for one head (or [B, H, S, d], evaluated head by head).
    Keys are consumed ``block`` at a time.  For each block: new running max =
    max(old max, block max); correction = exp(old max - new max), taken as 0
    while the old max is still -inf; l = correction * l + sum of the block's
    exp(score - new max); O = correction * O + (those weights) @ V_block.  After
    the last block O / l is the output.  ``trace``, if a list, receives
    (m, l, O_unnormalised, correction) copies after every block.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    if q.ndim == 4:
        B, H = q.shape[:2]
        outs = [[attention_tiled_ref(q[b, h], k[b, h], v[b, h], mask, window, scale, block)
                 for h in range(H)] for b in range(B)]
        o = np.stack([np.stack([x[0] for x in row]) for row in outs])
        lse = np.stack([np.stack([x[1] for x in row]) for row in outs])
        return o, lse
    S, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(S)
    m = np.full(S, -np.inf)
    l = np.zeros(S)
    acc = np.zeros((S, v.shape[-1]))
    for j0 in range(0, k.shape[0], block):
        cols = np.arange(j0, min(k.shape[0], j0 + block))
        s = scale * (q @ k[cols].T)
        s = np.where(visible(rows, cols, mask, window), s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = ~np.isneginf(m_new)
        with np.errstate(invalid="ignore"):
            corr = np.where(np.isneginf(m), 0.0, np.exp(m - np.where(live, m_new, 0.0)))
        p = np.exp(s - np.where(live, m_new, 0.0)[:, None])
        l = corr * l + p.sum(axis=1)
        acc = corr[:, None] * acc + p @ v[cols]
        m = m_new
        if trace is not None:
            trace.append((m.copy(), l.copy(), acc.copy(), corr.copy()))
    dead = np.isneginf(m)
    o = np.where(dead[:, None], 0.0, acc / np.where(dead, 1.0, l)[:, None])
    with np.errstate(divide="ignore"):
        lse = np.where(dead, -np.inf, m + np.log(np.where(dead, 1.0, l)))
    return o, lse


def attention_bwd_rows_ref(q, k, v, do, mask="none", window=None, scale=None):
    """Exact fp64 gradients of one head's attention, from the plain definition.

    q, k, v, do: [S, d] (do is the gradient of the loss with respect to O).
    Returns (dQ, dK, dV), each [S, d] fp64.

    The steps follow the Dev.to article's section "The backward pass: recompute
    instead of storing": with P the (materialised) softmax probabilities,
        dV = P^T dO,
        dP = dO V^T,
        dS = the softmax Jacobian applied to dP, row by row:
             dS[i, j] = P[i, j] * (dP[i, j] - sum_t P[i, t] dP[i, t]),
        dQ = scale * dS K,   dK = scale * dS^T Q
    (the last two are the matrix-product rules through S = scale * Q K^T).
    A row with no visible key has P = 0 and contributes nothing.
    """
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    S = q.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    rows = np.arange(S)
    s = scale * (q @ k.T)
    vis = visible(rows, np.arange(k.shape[0]), mask, window)
    s = np.where(vis, s, -np.inf)
    p, _, _ = _softmax_rows(s)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_bwd_ref(q, k, v, do, mask="none", window=None, scale=None, heads=None):
    """Exact fp64 gradients over [B, H, S, d] (K, V: [B, Hkv, S, d]; the
    gradient of a shared key/value head sums over its query heads).

    Returns (dQ [B,H,S,d], dK [B,Hkv,S,d], dV [B,Hkv,S,d]).  ``heads``
    optionally restricts the work to a list of (b, h) query heads (their
    contributions only; untouched entries of dQ are NaN).
    """
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    B, H, S, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, d) or v.shape[:3] != (B, Hkv, S) or do.shape[:3] != (B, H, S):
        raise ValueError("q, k, v, do shapes disagree")
    dq = np.full(q.shape, np.nan)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        g = kv_head(h, H, Hkv)
        dq[b, h], dk_h, dv_h = attention_bwd_rows_ref(q[b, h], k[b, g], v[b, g], do[b, h],
                                                      mask, window, scale)
        dk[b, g] += dk_h
        dv[b, g] += dv_h
    return dq, dk, dv

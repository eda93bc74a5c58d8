"""Tolerance of the backward parity tests: per-element error bounds of the
attention gradients when the inputs, the forward output and the two
intermediate operands P and dS are held in a 16-bit type and every product is
accumulated in fp32 (test infrastructure, not part of the library).

The bound is a first-order forward error analysis of the recomputation
backward pass (Dev.to, "FlashAttention: Why Tiling Attention Makes
Transformers Fast Without Changing the Result", section "The backward pass:
recompute instead of storing"), written with the exact fp64 quantities of one
head.  Notation: u is the unit roundoff of the element type (bf16 2^-8, fp16
2^-11), e = 2^-24 that of fp32, g = (S + d + 16) e a generous fp32
accumulation factor, |X| the elementwise absolute value, and a rounded
16-bit value x~ = x (1 + t) with |t| <= u (plus 2^-25 absolute for fp16
subnormals).  Step by step:

  forward output O~ (16-bit): |dO| <= u |O| + (u + g) |P| |V|
  row term D_i = dO_i . O~_i:  |dD| <= |dO| |dO_err| + g |dO||O|   (row sums)
  dP = dO V^T (fp32):          |d dP| <= g |dO| |V|^T
  P = exp(scale s - lse):      |dP_| <= P (|scale| g |Q||K|^T + g (1 + |lse|) + 4e)
  dS = P (dP - D), then ~:     |d dS| <= |dP_| |dP - D| + P (|d dP| + |dD|) + u |dS|
  dV = P~^T dO:                |d dV| <= ((u + g) P + |dP_|)^T |dO|
  dK = scale dS~^T Q:          |d dK| <= |scale| (|d dS| + g |dS|)^T |Q|
  dQ = scale dS~ K:            |d dQ| <= |scale| (|d dS| + g |dS|) |K|
and each gradient is rounded once more on output (+ u |grad|, and for fp16
+ 2^-25 absolute, the rounding error of a subnormal result).  These are
worst-case sums (all errors aligned), so real errors sit well below them; the
tests also check that plausible mistakes (a mask off by one, a missing row
term, a dropped scale, a tile left out) exceed them.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention_bwd_rows_ref, attention_probs_ref

UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
F32 = 2.0 ** -24


def _f64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def head_bounds(q, k, v, do, mask, window, scale, dtype):
    """Bounds before the final output rounding for one head ([S, d] inputs).

    Returns (eq, ek, ev) as [S, d] fp64 arrays: the bound on dQ's error, and
    this head's contributions to the bounds on dK and dV.
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    S, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    u = UNIT[dtype]
    sub = 2.0 ** -25 if dtype == "f16" else 0.0  # fp16 subnormal spacing / 2
    g = (S + d + 16) * F32
    p, m, l = attention_probs_ref(q, k, mask, window, scale)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), 0.0)
    o = p @ v
    dp = do @ v.T
    dd = (do * o).sum(axis=1)
    ds = p * (dp - dd[:, None])
    ado, av, aq, ak = np.abs(do), np.abs(v), np.abs(q), np.abs(k)
    pv = p @ av
    e_o = u * np.abs(o) + (u + g) * pv + sub
    e_d = (ado * e_o).sum(axis=1) + g * (ado * np.abs(o)).sum(axis=1)
    e_dp = g * (ado @ av.T)
    e_pr = p * (abs(scale) * g * (aq @ ak.T) + g * (1.0 + np.abs(lse))[:, None] + 4 * F32)
    e_ds = e_pr * np.abs(dp - dd[:, None]) + p * (e_dp + e_d[:, None]) + u * np.abs(ds)
    e_ds += sub * (p > 0)
    ev = (((u + g) * p + e_pr + sub * (p > 0)).T) @ ado
    w = e_ds + g * np.abs(ds)
    ek = abs(scale) * (w.T @ aq)
    eq = abs(scale) * (w @ ak)
    return eq, ek, ev


def grad_bounds(q, k, v, do, mask, window, scale, dtype):
    """Exact gradients and their error bounds over [B, H, S, d] (k, v:
    [B, Hkv, S, d]; query head h uses key/value head h // (H // Hkv)).

    Returns ((dq, dk, dv), (bq, bk, bv)), all fp64.
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    B, H, S, d = q.shape
    Hkv = k.shape[1]
    grp = H // Hkv
    u = UNIT[dtype]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    bq = np.zeros(q.shape)
    bk = np.zeros(k.shape)
    bv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            gh = h // grp
            args = (q[b, h], k[b, gh], v[b, gh], do[b, h], mask, window, scale)
            gq, gk, gv = attention_bwd_rows_ref(*args)
            eq, ek, ev = head_bounds(*args, dtype)
            dq[b, h] = gq
            dk[b, gh] += gk
            dv[b, gh] += gv
            bq[b, h] = eq
            bk[b, gh] += ek
            bv[b, gh] += ev
    # final rounding of each gradient (fp16 results below 2^-14 are subnormal:
    # their rounding error is absolute, at most 2^-25)
    sub = 2.0 ** -25 if dtype == "f16" else 0.0
    bq += u * np.abs(dq) + sub
    bk += u * np.abs(dk) + sub
    bv += u * np.abs(dv) + sub
    return (dq, dk, dv), (bq, bk, bv)


def excess(got, ref, bound):
    """max over elements of |got - ref| / bound (<= 1 means within the bound)."""
    err = np.abs(_f64(got) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / bound)
    return float(np.nanmax(r)) if r.size else 0.0

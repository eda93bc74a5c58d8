"""The backward tolerance (tests/bwd_bounds.py) is neither too tight nor too
loose: gradients computed with 16-bit rounding at the points where the
kernels round stay inside it, and plausible mistakes leave it.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

from bwd_bounds import UNIT, excess, grad_bounds
from oracle import attention_probs_ref
from workloads import make_grad, make_inputs

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _round(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(TDT[dtype]).double().numpy()


def _f64(t):
    return t.double().numpy()


def _case(dtype, mask, S=96, d=64, H=2, Hkv=2, window=None, seed=5):
    q, k, v = make_inputs(1, H, S, d, dtype, seed, Hkv=Hkv)
    do = make_grad(1, H, S, d, dtype, seed + 100)
    scale = 1.0 / math.sqrt(d)
    return q, k, v, do, scale


def _grads(q, k, v, do, mask, window, scale, dtype, mutate=None):
    """Gradients of one configuration with rounding at the kernels' points
    (P and dS to 16 bits before their products, the forward output and each
    gradient to 16 bits); ``mutate`` plants one mistake."""
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    B, H, S, d = q.shape
    Hkv = k.shape[1]
    grp = H // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for h in range(H):
        g = h // grp
        qh, kh, vh, doh = q[0, h], k[0, g], v[0, g], do[0, h]
        m_mask = mask
        if mutate == "mask_shift":  # causal boundary off by one (sees key i + 1)
            p, _, _ = attention_probs_ref(qh, np.vstack([kh[1:], kh[:1]]), mask, window, scale)
            p = np.hstack([p[:, -1:], p[:, :-1]])
        else:
            p, _, _ = attention_probs_ref(qh, kh, m_mask, window, scale)
        o = _round(_round(p, dtype) @ vh, dtype)
        dd = (doh * o).sum(axis=1)
        if mutate == "no_row_term":
            dd = 0 * dd
        dp = doh @ vh.T
        if mutate == "diag_leak":  # scores above the diagonal of one block not masked
            s = scale * (qh @ kh.T)
            lse = np.log(np.exp(np.where(p > 0, s, -np.inf)).sum(axis=1))
            leak = np.exp(s - lse[:, None])
            blk = np.zeros_like(p, dtype=bool)
            blk[32:64, 32:64] = True
            p = np.where(blk & (p == 0), leak, p)
        ds = _round(p * (dp - dd[:, None]), dtype)
        pr = _round(p, dtype)
        if mutate == "drop_tile":  # one 32-row query tile missing from dK, dV
            pr[32:64] = 0
            ds_kv = ds.copy()
            ds_kv[32:64] = 0
        else:
            ds_kv = ds
        sc_k = 1.0 if mutate == "no_scale" else scale
        dv[0, g] += pr.T @ doh
        dk[0, g] += sc_k * (ds_kv.T @ qh)
        if mutate == "transposed":
            dk[0, g] += scale * (ds @ qh) - scale * (ds_kv.T @ qh)
        dq[0, h] = _round(scale * (ds @ kh), dtype)
    return dq, _round(dk, dtype), _round(dv, dtype)


CASES = [("bf16", "causal", 2, None, 96), ("bf16", "none", 2, None, 96),
         ("f16", "causal", 2, None, 96), ("bf16", "window", 2, 40, 96),
         ("bf16", "causal", 1, None, 96), ("f16", "none", 1, None, 96),
         # the last keys of a causal sequence are seen by few rows: tiny dV
         # values, subnormal in fp16
         ("f16", "causal", 2, None, 129), ("f16", "causal", 1, None, 300)]


@pytest.mark.parametrize("dtype,mask,Hkv,window,S", CASES)
def test_rounded_gradients_stay_inside_the_bound(dtype, mask, Hkv, window, S):
    q, k, v, do, scale = _case(dtype, mask, S=S, Hkv=Hkv, window=window)
    ref, bnd = grad_bounds(q, k, v, do, mask, window, scale, dtype)
    got = _grads(q, k, v, do, mask, window, scale, dtype)
    for name, g, r, b in zip(("dq", "dk", "dv"), got, ref, bnd):
        x = excess(g, r, b)
        assert x <= 1.0, f"{name}: error reaches {x:.3f} of the bound"
        # and the rounding is visible at all (the bound is not vacuous)
        assert np.abs(g - r).max() > 0


@pytest.mark.parametrize("mutate", ["mask_shift", "no_row_term", "diag_leak", "drop_tile",
                                    "no_scale", "transposed"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_plausible_mistakes_leave_the_bound(mutate, dtype):
    mask = "causal"
    q, k, v, do, scale = _case(dtype, mask)
    ref, bnd = grad_bounds(q, k, v, do, mask, None, scale, dtype)
    got = _grads(q, k, v, do, mask, None, scale, dtype, mutate=mutate)
    worst = max(excess(g, r, b) for g, r, b in zip(got, ref, bnd))
    assert worst > 1.0, f"{mutate}: stays inside the bound ({worst:.3f})"


def test_bound_scales_with_the_unit_roundoff():
    q, k, v, do, scale = _case("bf16", "causal")
    _, b16 = grad_bounds(q, k, v, do, "causal", None, scale, "bf16")
    _, bh = grad_bounds(q, k, v, do, "causal", None, scale, "f16")
    ratio = UNIT["bf16"] / UNIT["f16"]
    for a, b in zip(b16, bh):
        r = np.median(a / b)
        assert 0.5 * ratio < r <= ratio * 1.01

"""Pins for the fp64 backward-pass oracle (gradients of exact attention).

The oracle's gradients are checked against things that do not come from it:
torch's autograd through its own fp64 scaled_dot_product_attention, central
finite differences of the (separately pinned) forward oracle, closed forms of
special cases, and an identity the page's recipe rests on.  Planted mistakes
in copies of the gradient formulas must be rejected.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_bwd_rows_ref, attention_ref, visible


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _vis(S, mask, window):
    return visible(np.arange(S), np.arange(S), mask, window)


def _torch_grads(q, k, v, do, mask, window, scale, gqa=False):
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    S = q.shape[2]
    kw = dict(scale=scale, enable_gqa=gqa)
    if mask == "causal":
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, **kw)
    else:
        m = torch.from_numpy(_vis(S, mask, window))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, **kw)
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 4)])
@pytest.mark.parametrize("S,d", [(1, 4), (9, 3), (40, 16)])
def test_gradients_against_torch_autograd_fp64(mask, window, S, d):
    B, H, scale = 2, 2, 1.0 / math.sqrt(d)
    q, k, v, do = (_rand((B, H, S, d), 80 + i) for i in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, mask, window, scale)
    tq, tk, tv = _torch_grads(q, k, v, do, mask, window, scale)
    np.testing.assert_allclose(dq, tq, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv, atol=1e-11, rtol=0)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (3, 3)])
def test_grouped_head_gradients_against_torch_autograd(H, Hkv):
    B, S, d, scale = 1, 13, 8, 0.3
    q, do = _rand((B, H, S, d), 90), _rand((B, H, S, d), 91)
    k, v = _rand((B, Hkv, S, d), 92), _rand((B, Hkv, S, d), 93)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, "causal", None, scale)
    tq, tk, tv = _torch_grads(q, k, v, do, "causal", None, scale, gqa=True)
    np.testing.assert_allclose(dq, tq, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk, atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv, atol=1e-11, rtol=0)


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 3)])
def test_gradients_against_central_finite_differences(mask, window):
    # L(Q, K, V) = sum(dO * O); its derivative is what the backward returns.
    S, d, scale, eps = 6, 3, 0.7, 1e-6
    q, k, v, do = (_rand((1, 1, S, d), 100 + i) for i in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, mask, window, scale)

    def loss(qq, kk, vv):
        o, _ = attention_ref(qq, kk, vv, mask, window, scale)
        return float((o * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                        loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=0, err_msg=name)


def test_window_of_one_closed_form():
    # Every query sees only its own key: O = V, independent of Q and K.
    S, d = 11, 5
    q, k, v, do = (_rand((S, d), 110 + i) for i in range(4))
    dq, dk, dv = attention_bwd_rows_ref(q, k, v, do, "window", 1, 0.4)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, do)


def test_zero_keys_closed_form():
    # K = 0: every visible key gets weight 1/n_i; dV_j = sum over rows i that
    # see j of dO_i / n_i, and dK_j = scale * sum_i dS_ij q_i with
    # dS_ij = (dO_i . v_j - dO_i . O_i) / n_i on visible pairs.
    S, d, scale = 9, 4, 0.5
    q, v, do = _rand((S, d), 120), _rand((S, d), 121), _rand((S, d), 122)
    k = np.zeros((S, d))
    dq, dk, dv = attention_bwd_rows_ref(q, k, v, do, "causal", None, scale)
    n = np.arange(1, S + 1, dtype=np.float64)
    want_dv = np.zeros((S, d))
    for j in range(S):
        for i in range(j, S):
            want_dv[j] += do[i] / n[i]
    np.testing.assert_allclose(dv, want_dv, atol=1e-13)
    o = np.cumsum(v, axis=0) / n[:, None]
    want_dk = np.zeros((S, d))
    for i in range(S):
        for j in range(i + 1):
            want_dk[j] += scale * (do[i] @ v[j] - do[i] @ o[i]) / n[i] * q[i]
    np.testing.assert_allclose(dk, want_dk, atol=1e-13)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)  # dQ = scale * dS K, K = 0


def test_softmax_jacobian_row_term_equals_do_dot_o():
    # The Jacobian's row term sum_t P[i,t] dP[i,t] equals dO_i . O_i, which is
    # what lets a kernel compute it from O instead of from P.
    S, d, scale = 17, 6, 0.3
    q, k, v, do = (_rand((1, 1, S, d), 130 + i) for i in range(4))
    o, _ = attention_ref(q, k, v, "causal", None, scale)
    s = scale * q[0, 0] @ k[0, 0].T
    s = np.where(_vis(S, "causal", None), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose((p * dp).sum(axis=1), (do[0, 0] * o[0, 0]).sum(axis=1),
                               atol=1e-12)


def _mutant_grads(kind, q, k, v, do, mask, window, scale):
    S = q.shape[0]
    s = scale * q @ k.T
    s = np.where(_vis(S, mask, window), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dv = (p @ do) if kind == "dv_untransposed" else p.T @ do
    dp = do @ v.T
    ds = p * dp if kind == "no_row_term" else p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * ds @ k
    dk = (ds.T @ q) if kind == "dk_without_scale" else scale * ds.T @ q
    if kind == "dq_from_dst":
        dq = scale * ds.T @ k
    return dq, dk, dv


@pytest.mark.parametrize("kind", ["dv_untransposed", "no_row_term", "dk_without_scale",
                                  "dq_from_dst"])
def test_pins_reject_planted_gradient_mistakes(kind):
    S, d, scale = 10, 4, 0.6
    q, k, v, do = (_rand((1, 1, S, d), 140 + i) for i in range(4))
    got = _mutant_grads(kind, q[0, 0], k[0, 0], v[0, 0], do[0, 0], "causal", None, scale)
    want = _torch_grads(q, k, v, do, "causal", None, scale)
    assert not all(np.allclose(g, w[0, 0], atol=1e-8) for g, w in zip(got, want))
    # ... and the oracle itself passes the same pin
    mine = attention_bwd_rows_ref(q[0, 0], k[0, 0], v[0, 0], do[0, 0], "causal", None, scale)
    assert all(np.allclose(g, w[0, 0], atol=1e-11) for g, w in zip(mine, want))

"""Pins for the fp64 oracle, checked against facts that do not come from it.

Each test fixes the oracle to something other than itself: values printed on
the pages for their worked examples (fixtures under tests/golden/ carry the
citation), closed forms and special cases of the definition, invariants the
pages state, a library routine (torch's fp64 scaled_dot_product_attention and
scipy's logsumexp), and a high-precision brute force on tiny inputs.  The last
group plants plausible mistakes into copies of the oracle and checks that at
least one pin rejects each of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

from oracle import (attention_probs_ref, attention_ref, attention_rows_ref,
                    attention_tiled_ref, kv_head, visible)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# the pages' worked examples
# --------------------------------------------------------------------------

def test_worked_example_direct():
    g = _load("worked_example_tiles.json")
    q = np.array([g["q"]])
    K, V = np.array(g["K"]), np.array(g["V"])
    P, m, l = attention_probs_ref(q, K, scale=g["scale"])
    np.testing.assert_allclose(P[0], g["probs"], atol=g["probs_tol"])
    assert abs(P[0].sum() - 1.0) < 1e-15
    o, lse = attention_rows_ref(q, K, V, [0], scale=g["scale"])
    np.testing.assert_allclose(o[0], g["O_final"], atol=g["O_final_tol"])
    # the scores are integers, so the max-shifted denominator is a closed form
    l_exact = sum(math.exp(s - 3.0) for s in g["scores"])
    assert abs(l[0] - l_exact) < 1e-15 and m[0] == 3.0
    assert abs(lse[0] - (3.0 + math.log(l_exact))) < 1e-14
    # V's second column is its first plus one, so O's is too (printed output)
    assert abs((o[0, 1] - o[0, 0]) - 1.0) < 1e-14


def test_worked_example_tiled_trace():
    g = _load("worked_example_tiles.json")
    q = np.array([g["q"]])
    K, V = np.array(g["K"]), np.array(g["V"])
    trace = []
    o, lse = attention_tiled_ref(q, K, V, scale=g["scale"], block=g["block"], trace=trace)
    assert len(trace) == len(g["tiles"])
    for (m, l, acc, corr), want in zip(trace, g["tiles"]):
        assert abs(m[0] - want["m"]) < 1e-15
        assert abs(l[0] - want["l"]) < g["trace_tol"]
        np.testing.assert_allclose(acc[0], want["O_unnormalised"], atol=g["trace_tol"])
        assert abs(corr[0] - want["correction"]) < g["trace_tol"]
    np.testing.assert_allclose(o[0], g["O_final"], atol=g["O_final_tol"])


def test_worked_example_single_block():
    g = _load("worked_example_tiles.json")
    sb = g["single_block"]
    q = np.array([g["q"]])
    K, V = np.array(g["K"]), np.array(g["V"])
    trace = []
    o, _ = attention_tiled_ref(q, K, V, scale=g["scale"], block=sb["block"], trace=trace)
    assert len(trace) == 1
    m, l, acc, corr = trace[0]
    assert m[0] == sb["m"] and corr[0] == 0.0
    assert abs(l[0] - sb["l"]) < sb["l_tol"]
    np.testing.assert_allclose(o[0], g["O_final"], atol=g["O_final_tol"])
    # unnormalised weights of the single block
    p = np.exp(np.array(g["scores"]) - sb["m"])
    np.testing.assert_allclose(p, sb["p_unnormalised"], atol=sb["p_tol"])


def test_two_block_row_example():
    g = _load("two_block_row.json")
    s = np.array(g["scores"])
    q = np.array([[1.0]])
    K = s[:, None]
    V = np.eye(4)  # O then equals the probability row itself
    trace = []
    o, lse = attention_tiled_ref(q, K, V, scale=1.0, block=g["block"], trace=trace)
    (m1, l1, _, _), (m2, l2, _, c2) = trace
    tol = g["tol"]
    assert m1[0] == g["block1_max"] and m2[0] == g["final_max"]
    assert abs(l1[0] - g["block1_sum"]) < tol
    assert abs(c2[0] - g["rescale_factor"]) < tol
    assert abs(c2[0] * l1[0] - g["rescaled_sum"]) < tol
    assert abs(l2[0] - g["denominator"]) < tol
    P, _, l = attention_probs_ref(q, K, scale=1.0)
    assert abs(l[0] - g["denominator"]) < tol
    np.testing.assert_allclose(o[0], P[0], atol=1e-15)
    # both worked examples share the max-shifted multiset {0, -2, -3, -4}
    w = _load("worked_example_tiles.json")
    assert abs(l2[0] - w["tiles"][-1]["l"]) < 5e-5


# --------------------------------------------------------------------------
# invariants and closed forms of the definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 3)])
def test_probability_rows_sum_to_one(mask, window):
    q, k = _rand((13, 8), 1), _rand((13, 8), 2)
    P, m, l = attention_probs_ref(q, k, mask, window, scale=0.7)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    assert (P >= 0).all()
    vis = visible(np.arange(13), np.arange(13), mask, window)
    assert (P[~vis] == 0).all() and (P[vis] > 0).all()


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 4)])
def test_output_in_convex_hull_of_visible_values(mask, window):
    S, d = 17, 6
    q, k, v = _rand((1, 1, S, d), 3), _rand((1, 1, S, d), 4), _rand((1, 1, S, d), 5)
    o, _ = attention_ref(q, k, v, mask, window)
    vis = visible(np.arange(S), np.arange(S), mask, window)
    for i in range(S):
        vv = v[0, 0][vis[i]]
        assert (o[0, 0, i] >= vv.min(axis=0) - 1e-12).all()
        assert (o[0, 0, i] <= vv.max(axis=0) + 1e-12).all()


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 5)])
def test_zero_keys_give_mean_of_visible_values(mask, window):
    S, d = 12, 4
    q, v = _rand((1, 1, S, d), 6), _rand((1, 1, S, d), 7)
    k = np.zeros_like(q)
    o, lse = attention_ref(q, k, v, mask, window, scale=0.3)
    vis = visible(np.arange(S), np.arange(S), mask, window)
    for i in range(S):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0][vis[i]].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(vis[i].sum())) < 1e-14


def test_causal_first_row_is_first_value():
    S, d, scale = 9, 5, 0.37
    q, k, v = _rand((2, 3, S, d), 8), _rand((2, 3, S, d), 9), _rand((2, 3, S, d), 10)
    o, lse = attention_ref(q, k, v, "causal", scale=scale)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], scale * (q[:, :, 0] * k[:, :, 0]).sum(-1),
                               atol=1e-14)


def test_window_one_is_identity():
    S, d, scale = 11, 3, 1.3
    q, k, v = _rand((1, 2, S, d), 11), _rand((1, 2, S, d), 12), _rand((1, 2, S, d), 13)
    o, lse = attention_ref(q, k, v, "window", 1, scale=scale)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, scale * (q * k).sum(-1), atol=1e-14)


def test_window_covering_sequence_equals_causal():
    S, d = 10, 4
    q, k, v = _rand((1, 1, S, d), 14), _rand((1, 1, S, d), 15), _rand((1, 1, S, d), 16)
    oc, lc = attention_ref(q, k, v, "causal")
    for W in (S, S + 1, 10 * S):
        ow, lw = attention_ref(q, k, v, "window", W)
        np.testing.assert_array_equal(ow, oc)
        np.testing.assert_array_equal(lw, lc)


def test_window_counts_the_diagonal():
    vis = visible(np.arange(6), np.arange(6), "window", 2)
    want = np.array([[j in (i - 1, i) for j in range(6)] for i in range(6)])
    np.testing.assert_array_equal(vis, want)
    assert visible(np.arange(6), np.arange(6), "causal", None).sum() == 21


def test_constant_value_column_gives_constant_output_column():
    S, d = 14, 4
    q, k, v = _rand((1, 1, S, d), 17), _rand((1, 1, S, d), 18), _rand((1, 1, S, d), 19)
    v[..., 2] = 3.25
    for mask, W in (("none", None), ("causal", None), ("window", 3)):
        o, _ = attention_ref(q, k, v, mask, W)
        np.testing.assert_allclose(o[..., 2], 3.25, atol=1e-14)


def test_permutation_equivariance_without_mask():
    S, d = 15, 5
    q, k, v = _rand((1, 1, S, d), 20), _rand((1, 1, S, d), 21), _rand((1, 1, S, d), 22)
    o, lse = attention_ref(q, k, v)
    perm = np.random.default_rng(0).permutation(S)
    o2, lse2 = attention_ref(q, k[:, :, perm], v[:, :, perm])   # same keys, new order
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)
    o3, lse3 = attention_ref(q[:, :, perm], k, v)                # queries permute O
    np.testing.assert_allclose(o3, o[:, :, perm], atol=1e-14)
    np.testing.assert_allclose(lse3, lse[:, :, perm], atol=1e-14)


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 4)])
def test_score_shift_moves_lse_not_output(mask, window):
    """Adding c to every score leaves O alone and adds c to the LSE.

    Realised by an extra feature: q' = [q, c / scale], k' = [k, 1].
    """
    S, d, scale, c = 13, 4, 0.5, 7.25
    q, k, v = _rand((1, 1, S, d), 23), _rand((1, 1, S, d), 24), _rand((1, 1, S, d), 25)
    o, lse = attention_ref(q, k, v, mask, window, scale=scale)
    q2 = np.concatenate([q, np.full((1, 1, S, 1), c / scale)], -1)
    k2 = np.concatenate([k, np.ones((1, 1, S, 1))], -1)
    o2, lse2 = attention_ref(q2, k2, v, mask, window, scale=scale)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + c, atol=1e-13)


def test_huge_scores_do_not_overflow():
    """Max subtraction keeps exp bounded: scores near 1e4 still give a finite,
    essentially one-hot result."""
    S, d = 16, 8
    q, k, v = _rand((1, 1, S, d), 26), _rand((1, 1, S, d), 27), _rand((1, 1, S, d), 28)
    o, lse = attention_ref(q, k, v, scale=2000.0)
    s = 2000.0 * q[0, 0] @ k[0, 0].T
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    top = s.argmax(axis=1)
    gap = np.sort(s, axis=1)[:, -1] - np.sort(s, axis=1)[:, -2]
    ok = gap > 50  # rows whose winner is clear by e^-50
    np.testing.assert_allclose(o[0, 0][ok], v[0, 0][top[ok]], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0][ok], s.max(axis=1)[ok], atol=1e-12)


def test_row_chunking_does_not_change_result():
    S, d = 40, 4
    q, k, v = _rand((1, 2, S, d), 29), _rand((1, 2, S, d), 30), _rand((1, 2, S, d), 31)
    o1, l1 = attention_ref(q, k, v, "window", 9, row_chunk=2048)
    o2, l2 = attention_ref(q, k, v, "window", 9, row_chunk=7)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


# --------------------------------------------------------------------------
# one-pass vs tiled (block size never changes the result)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 1),
                                         ("window", 5), ("window", 100)])
def test_tiled_equals_one_pass_for_every_block_size(mask, window):
    S, d = 19, 6
    q = _rand((S, d), 32, 2.0)
    k = _rand((S, d), 33, 2.0)
    v = _rand((S, d), 34)
    o, lse = attention_rows_ref(q, k, v, np.arange(S), mask, window, scale=0.8)
    for block in range(1, S + 1):
        ot, lt = attention_tiled_ref(q, k, v, mask, window, scale=0.8, block=block)
        np.testing.assert_allclose(ot, o, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lt, lse, atol=1e-12, rtol=0)


def test_tiled_running_max_never_decreases_and_correction_at_most_one():
    S, d = 24, 4
    q, k, v = _rand((S, d), 35, 3.0), _rand((S, d), 36, 3.0), _rand((S, d), 37)
    trace = []
    attention_tiled_ref(q, k, v, "none", scale=1.0, block=5, trace=trace)
    prev = np.full(S, -np.inf)
    for m, l, acc, corr in trace:
        assert (m >= prev).all()
        assert (corr <= 1.0).all() and (corr >= 0.0).all()
        prev = m


# --------------------------------------------------------------------------
# library routines and high-precision brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 6)])
@pytest.mark.parametrize("S,d", [(1, 4), (7, 3), (33, 16), (64, 64)])
def test_against_torch_sdpa_fp64(mask, window, S, d):
    B, H, scale = 2, 3, 1.0 / math.sqrt(d)
    q, k, v = _rand((B, H, S, d), 38), _rand((B, H, S, d), 39), _rand((B, H, S, d), 40)
    o, lse = attention_ref(q, k, v, mask, window, scale=scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    if mask == "causal":
        want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                                scale=scale)
    else:
        vis = torch.from_numpy(visible_torchless(S, mask, window))
        want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=vis,
                                                                scale=scale)
    np.testing.assert_allclose(o, want.numpy(), atol=1e-12, rtol=0)
    scores = torch.matmul(tq, tk.transpose(-1, -2).contiguous()).numpy() * scale
    vis = visible_torchless(S, mask, window)
    scores = np.where(vis, scores, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(scores, axis=-1), atol=1e-12)


def visible_torchless(S, mask, window):
    """Visibility written independently of the oracle (for the library check)."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    if mask == "none":
        return np.ones((S, S), dtype=bool)
    if mask == "causal":
        return j <= i
    return (j <= i) & (i - j < window)


def _mp_attention(q, k, v, scale, vis):
    mpmath.mp.dps = 50
    S, d = q.shape
    o = np.zeros((S, v.shape[1]))
    lse = np.zeros(S)
    for i in range(S):
        sc = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i, t]) * mpmath.mpf(k[j, t])
                                              for t in range(d))
              for j in range(S) if vis[i, j]]
        js = [j for j in range(S) if vis[i, j]]
        w = [mpmath.exp(s) for s in sc]          # no shift needed at 50 digits
        tot = mpmath.fsum(w)
        for c in range(v.shape[1]):
            o[i, c] = float(mpmath.fsum(wi * mpmath.mpf(v[j, c]) for wi, j in zip(w, js)) / tot)
        lse[i] = float(mpmath.log(tot))
    return o, lse


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 3)])
def test_brute_force_mpmath(mask, window):
    S, d, scale = 10, 5, 0.6
    q, k, v = _rand((S, d), 41, 1.5), _rand((S, d), 42, 1.5), _rand((S, d), 43)
    o, lse = attention_rows_ref(q, k, v, np.arange(S), mask, window, scale)
    o_mp, lse_mp = _mp_attention(q, k, v, scale, visible_torchless(S, mask, window))
    np.testing.assert_allclose(o, o_mp, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, lse_mp, atol=1e-13, rtol=0)


# --------------------------------------------------------------------------
# grouped key/value heads (query head h uses key/value head h // (H / Hkv))
# --------------------------------------------------------------------------

def _sdpa_gqa(q, k, v, mask, window, scale):
    """torch's own grouped-query attention (enable_gqa) in fp64, plus the
    logsumexp of the visible scaled scores through scipy."""
    S = q.shape[2]
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    if mask == "causal":
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                            scale=scale, enable_gqa=True)
    else:
        vis = torch.from_numpy(visible_torchless(S, mask, window))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=vis,
                                                            scale=scale, enable_gqa=True)
    group = q.shape[1] // k.shape[1]
    kr = torch.repeat_interleave(tk, group, dim=1)
    scores = torch.matmul(tq, kr.transpose(-1, -2).contiguous()).numpy() * scale
    scores = np.where(visible_torchless(S, mask, window), scores, -np.inf)
    return o.numpy(), scipy.special.logsumexp(scores, axis=-1)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 3), (4, 1), (8, 4), (3, 3)])
@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None), ("window", 5)])
def test_grouped_heads_against_torch_sdpa_fp64(H, Hkv, mask, window):
    B, S, d = 2, 19, 8
    scale = 1.0 / math.sqrt(d)
    q = _rand((B, H, S, d), 60)
    k, v = _rand((B, Hkv, S, d), 61), _rand((B, Hkv, S, d), 62)
    o, lse = attention_ref(q, k, v, mask, window, scale=scale)
    want_o, want_lse = _sdpa_gqa(q, k, v, mask, window, scale)
    np.testing.assert_allclose(o, want_o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, want_lse, atol=1e-12, rtol=0)


def test_grouped_heads_share_their_key_value_head():
    # Query heads of one group that carry the same queries give the same rows;
    # heads of different groups differ.
    B, H, Hkv, S, d = 1, 6, 2, 11, 4
    q1 = _rand((1, 1, S, d), 63)
    q = np.repeat(q1, H, axis=1)
    k, v = _rand((B, Hkv, S, d), 64), _rand((B, Hkv, S, d), 65)
    o, lse = attention_ref(q, k, v, "causal")
    for h in range(H):
        assert kv_head(h, H, Hkv) == h // 3
        np.testing.assert_array_equal(o[0, h], o[0, 3 * (h // 3)])
    assert not np.allclose(o[0, 0], o[0, 3])


def test_grouped_heads_reject_non_dividing_counts():
    q, k = _rand((1, 4, 5, 2), 66), _rand((1, 3, 5, 2), 67)
    with pytest.raises(ValueError):
        attention_ref(q, k, k)
    with pytest.raises(ValueError):
        kv_head(0, 4, 0)


def test_grouped_heads_reject_wrong_head_mapping():
    # A plausible mistake (interleaved instead of contiguous groups) is caught
    # by the torch pin.
    B, H, Hkv, S, d = 1, 4, 2, 7, 4
    q = _rand((B, H, S, d), 68)
    k, v = _rand((B, Hkv, S, d), 69), _rand((B, Hkv, S, d), 70)
    want_o, _ = _sdpa_gqa(q, k, v, "none", None, 0.5)
    wrong = np.stack([attention_rows_ref(q[0, h], k[0, h % Hkv], v[0, h % Hkv], np.arange(S),
                                         "none", None, 0.5)[0] for h in range(H)])[None]
    assert not np.allclose(wrong, want_o, atol=1e-6)


# --------------------------------------------------------------------------
# planted mistakes: each must be rejected by at least one pin above
# --------------------------------------------------------------------------

def _pins_pass(rows_ref):
    """A compact re-run of pins that do not depend on the oracle's own output,
    driven through a candidate ``rows_ref(q, k, v, rows, mask, window, scale)``."""
    g = _load("worked_example_tiles.json")
    q = np.array([g["q"]])
    K, V = np.array(g["K"]), np.array(g["V"])
    try:
        o, lse = rows_ref(q, K, V, [0], "none", None, 1.0)
        if not np.allclose(o[0], g["O_final"], atol=1e-8):
            return False
        if abs(lse[0] - (3.0 + math.log(sum(math.exp(s - 3) for s in g["scores"])))) > 1e-12:
            return False
        S, d, scale = 9, 4, 0.37
        qq, kk, vv = _rand((S, d), 50), _rand((S, d), 51), _rand((S, d), 52)
        o, lse = rows_ref(qq, kk, vv, np.arange(S), "causal", None, scale)
        if not np.allclose(o[0], vv[0], atol=1e-14):
            return False
        if abs(lse[0] - scale * qq[0] @ kk[0]) > 1e-14:
            return False
        o, _ = rows_ref(qq, kk, vv, np.arange(S), "window", 1, scale)
        if not np.allclose(o, vv, atol=1e-14):
            return False
        o, lse = rows_ref(qq, np.zeros_like(kk), vv, np.arange(S), "causal", None, scale)
        if not np.allclose(lse, np.log(np.arange(1, S + 1)), atol=1e-14):
            return False
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (qq, kk, vv))
        want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        o, _ = rows_ref(qq, kk, vv, np.arange(S), "none", None, scale)
        if not np.allclose(o, want[0, 0].numpy(), atol=1e-12):
            return False
    except (ValueError, IndexError, FloatingPointError):
        return False
    return True


def _mutant(kind):
    def rows_ref(q, k, v, rows, mask, window, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        rows = np.asarray(rows)
        s = q[rows] @ k.T
        if kind != "drop_scale":
            s = s * scale
        cols = np.arange(k.shape[0])
        if kind == "mask_flipped" and mask != "none":
            vis = cols[None, :] >= rows[:, None]
        elif kind == "window_off_by_one" and mask == "window":
            vis = (cols[None, :] <= rows[:, None]) & (cols[None, :] >= rows[:, None] - window)
        else:
            vis = visible(rows, cols, mask, window)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        sign = -1.0 if kind == "wrong_sign" else 1.0
        e = np.exp(sign * (s - m[:, None]))
        e = np.where(vis, e, 0.0)
        l = e.sum(axis=1)
        p = e / l[:, None]
        vv = v.T if kind == "transposed_v" else v
        o = p @ vv
        lse = m + (np.log2(l) if kind == "log2_lse" else np.log(l))
        if kind == "lse_without_max":
            lse = np.log(l)
        return o, lse
    return rows_ref


def test_pins_accept_the_oracle():
    assert _pins_pass(lambda q, k, v, r, m, w, s: attention_rows_ref(q, k, v, r, m, w, s))


@pytest.mark.parametrize("kind", ["drop_scale", "mask_flipped", "window_off_by_one",
                                  "wrong_sign", "transposed_v", "log2_lse",
                                  "lse_without_max"])
def test_pins_reject_planted_mistakes(kind):
    assert not _pins_pass(_mutant(kind))

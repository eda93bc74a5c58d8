"""Pins of the paged-cache decode oracle (oracle/decode.py) against things
other than itself: the chapter's printed block arithmetic, the causal prefill
definition, torch's attention, closed forms, invariances of the layout, and a
pure-Python loop on tiny inputs.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_ref, paged_decode_ref, paged_gather, paged_token_slots
from workloads import (DECODE_WORKLOADS, blocks_needed, generate_decode, kv_bytes_per_token,
                       make_decode_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_kv_example.json")


def _inputs(B=3, H=4, Hkv=2, n_q=2, d=16, bs=4, ctx=(9, 1, 13), seed=3, extra=3,
            dtype="bf16"):
    return make_decode_inputs(B, H, Hkv, n_q, d, dtype, bs, seed, ctx_lens=list(ctx),
                              extra_blocks=extra)


def _contiguous(cache, table_row, n, g):
    """The request's first n rows of head g, in logical order (via the oracle's
    own slot map, which the golden and layout tests pin separately)."""
    return paged_gather(cache, table_row, n, g)[1]


# -- the chapter's worked numbers ------------------------------------------

def test_page_example_block_arithmetic():
    ex = json.load(open(GOLDEN))
    m = ex["model"]
    # 2 (K and V) x layers x hidden x bytes: the hidden size is heads x d
    assert kv_bytes_per_token(m["hidden"] // 128, 128, m["bytes_per_value"],
                              layers=m["layers"]) == ex["kv_per_token_bytes"]
    bs, n = ex["block_size"], ex["actual_tokens"]
    assert blocks_needed(n, bs) == ex["blocks_needed"]
    # a 90-token request scattered over six physical blocks of a larger pool
    table = np.array([41, 7, 19, 3, 30, 12, -1, -1])
    pos, blocks, slots = paged_token_slots(table, n, bs, num_blocks=64)
    assert list(pos) == list(range(n))
    assert len(set(blocks.tolist())) == ex["blocks_needed"]
    reserved_slots = len(set(blocks.tolist())) * bs
    assert reserved_slots == ex["paged_slots"]
    assert round(100 * n / reserved_slots, 1) == ex["paged_util_pct"]
    assert round(100 * n / ex["max_context"], 1) == ex["naive_util_pct"]
    kv = ex["kv_per_token_bytes"]
    assert ex["max_context"] * kv / 2 ** 20 == ex["naive_reserved_MiB"]
    assert abs(reserved_slots * kv / 2 ** 20 - ex["paged_reserved_MiB_about"]) < 1
    # the partly filled last block: slots 0..9 of block 12 hold tokens 80..89
    last = blocks == 12
    assert slots[last].tolist() == list(range(10)) and pos[last].tolist() == list(range(80, 90))


# -- against the causal prefill definition and torch -------------------------

@pytest.mark.parametrize("bs", [1, 4, 16])
def test_all_new_tokens_is_causal_prefill(bs):
    """With every cached token a query row (n_q = n), decoding is exactly the
    causal prefill of the gathered sequence."""
    n = 23
    q, kc, vc, table, ctx = make_decode_inputs(1, 4, 2, n, 16, "f16", bs, 5, ctx_lens=[n],
                                               extra_blocks=4)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    k = torch.stack([torch.from_numpy(_contiguous(kc, table[0], n, g)) for g in range(2)])
    v = torch.stack([torch.from_numpy(_contiguous(vc, table[0], n, g)) for g in range(2)])
    o_ref, lse_ref = attention_ref(q.double(), k[None], v[None], "causal")
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_matches_torch_attention():
    q, kc, vc, table, ctx = _inputs()
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    B, H, n_q, d = q.shape
    group = H // kc.shape[1]
    for b in range(B):
        n = int(ctx[b])
        for h in range(H):
            g = h // group
            k = torch.from_numpy(_contiguous(kc, table[b], n, g))
            v = torch.from_numpy(_contiguous(vc, table[b], n, g))
            rows = n - n_q + torch.arange(n_q)
            vis = torch.arange(n)[None, :] <= rows[:, None]
            s = (q[b, h].double() @ k.T) / math.sqrt(d)
            for i in range(n_q):
                if not vis[i].any():
                    assert np.all(o[b, h, i] == 0) and lse[b, h, i] == -np.inf
                    continue
                ref = torch.nn.functional.scaled_dot_product_attention(
                    q[b, h, i:i + 1].double()[None], k[None], v[None],
                    attn_mask=vis[i:i + 1][None])
                np.testing.assert_allclose(o[b, h, i], ref[0, 0].numpy(), atol=1e-12)
                np.testing.assert_allclose(lse[b, h, i],
                                           torch.logsumexp(s[i][vis[i]], 0).item(), atol=1e-12)


def test_pure_python_loops_tiny():
    """An independent reading on a tiny case: dict page table, math.exp."""
    q, kc, vc, table, ctx = _inputs(B=2, H=2, Hkv=1, n_q=2, d=3, bs=2, ctx=(5, 3), seed=9)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx, scale=0.7)
    qf, kf, vf = q.double().tolist(), kc.double().tolist(), vc.double().tolist()
    for b in range(2):
        pages = {j: int(e) for j, e in enumerate(table[b].tolist())}
        n = int(ctx[b])
        for h in range(2):
            for i in range(2):
                last = n - 2 + i
                sc, vs = [], []
                for t in range(last + 1):
                    blk, slot = pages[t // 2], t % 2
                    key, val = kf[blk][0][slot], vf[blk][0][slot]
                    sc.append(0.7 * sum(a * c for a, c in zip(qf[b][h][i], key)))
                    vs.append(val)
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                for c in range(3):
                    assert abs(o[b, h, i, c] - sum(wi * vi[c] for wi, vi in zip(w, vs)) / tot) \
                        < 1e-12
                assert abs(lse[b, h, i] - (mx + math.log(tot))) < 1e-12


# -- closed forms -------------------------------------------------------------

def test_single_cached_token():
    q, kc, vc, table, ctx = _inputs(ctx=(1, 1, 1), n_q=1)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx, scale=0.3)
    for b in range(3):
        blk = int(table[b, 0])
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(o[b, h, 0], vc[blk, g, 0].double().numpy())
            ref = 0.3 * float(q[b, h, 0].double() @ kc[blk, g, 0].double())
            assert abs(lse[b, h, 0] - ref) < 1e-12


def test_zero_keys_average_the_visible_values():
    q, kc, vc, table, ctx = _inputs(ctx=(9, 4, 13), n_q=3)
    kc = torch.zeros_like(kc)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    for b in range(3):
        n = int(ctx[b])
        for h in range(4):
            v = _contiguous(vc, table[b], n, h // 2)
            for i in range(3):
                seen = n - 3 + i + 1
                np.testing.assert_allclose(o[b, h, i], v[:seen].mean(axis=0), atol=1e-12)
                assert abs(lse[b, h, i] - math.log(seen)) < 1e-12


# -- invariances of the layout -------------------------------------------------

def test_moving_blocks_changes_nothing():
    q, kc, vc, table, ctx = _inputs()
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    rng = np.random.default_rng(1)
    perm = rng.permutation(kc.shape[0])          # physical block p moves to perm[p]
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    kc2[torch.from_numpy(perm)] = kc
    vc2[torch.from_numpy(perm)] = vc
    t2 = table.clone()
    valid = t2 >= 0
    t2[valid] = torch.from_numpy(perm)[t2[valid].long()].to(t2.dtype)
    o2, lse2 = paged_decode_ref(q, kc2, vc2, t2, ctx)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("bs", [1, 3, 7, 32])
def test_block_size_does_not_matter(bs):
    """The same logical sequences stored with another block size."""
    q, kc, vc, table, ctx = _inputs(bs=4)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    B, Hkv = 3, 2
    need = [blocks_needed(int(n), bs) for n in ctx]
    kc2 = torch.zeros(sum(need), Hkv, bs, kc.shape[-1], dtype=kc.dtype)
    vc2 = torch.zeros_like(kc2)
    t2 = torch.full((B, max(need)), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        n = int(ctx[b])
        for j in range(need[b]):
            t2[b, j] = nxt + j
        for g in range(Hkv):
            k = torch.from_numpy(_contiguous(kc, table[b], n, g)).to(kc.dtype)
            v = torch.from_numpy(_contiguous(vc, table[b], n, g)).to(vc.dtype)
            for t in range(n):
                kc2[nxt + t // bs, g, t % bs] = k[t]
                vc2[nxt + t // bs, g, t % bs] = v[t]
        nxt += need[b]
    o2, lse2 = paged_decode_ref(q, kc2, vc2, t2, ctx)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_grouped_heads_equal_repeated_heads():
    q, kc, vc, table, ctx = _inputs(H=6, Hkv=2)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    kr, vr = kc.repeat_interleave(3, dim=1), vc.repeat_interleave(3, dim=1)
    o2, lse2 = paged_decode_ref(q, kr, vr, table, ctx)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # and a wrong mapping (h % Hkv) would differ
    kw = torch.cat([kc] * 3, dim=1)
    vw = torch.cat([vc] * 3, dim=1)
    o3, _ = paged_decode_ref(q, kw, vw, table, ctx)
    assert np.abs(o3 - o).max() > 1e-3


# -- table entries that hold no block, context lengths out of range ---------------

def test_shared_prefix_blocks_equal_private_copies():
    """Copy-on-write prefix sharing (aicomputerinstitute.com flash-attention
    chapter, "PagedAttention: memory management borrowed from an operating
    system"): several requests whose tables name the same physical blocks for
    a common prefix give exactly what they give with that prefix copied into
    blocks of their own, and a request sharing another's whole context (and
    query) reproduces that request's result."""
    q, kc, vc, table, ctx = make_decode_inputs(3, 4, 2, 1, 16, "bf16", 4, 5,
                                               ctx_lens=[30, 41, 30], extra_blocks=2)
    P = 5
    shared = table.clone()
    kc_own, vc_own = kc.clone(), vc.clone()
    for b in (1, 2):
        shared[b, :P] = table[0, :P]
        kc_own[table[b, :P].long()] = kc[table[0, :P].long()]
        vc_own[table[b, :P].long()] = vc[table[0, :P].long()]
    o_s, l_s = paged_decode_ref(q, kc, vc, shared, ctx)
    o_c, l_c = paged_decode_ref(q, kc_own, vc_own, table, ctx)
    assert np.array_equal(o_s, o_c) and np.array_equal(l_s, l_c)
    # request 2 shares all of request 0's blocks and its query: same result
    full = table.clone()
    full[2] = table[0]
    q2 = q.clone()
    q2[2] = q[0]
    o_f, l_f = paged_decode_ref(q2, kc, vc, full, ctx)
    assert np.array_equal(o_f[2], o_f[0]) and np.array_equal(l_f[2], l_f[0])
    # and sharing did change what request 1 sees (the prefix is not its own)
    assert not np.allclose(o_s[1], paged_decode_ref(q, kc, vc, table, ctx)[0][1])


def test_invalid_entries_hold_no_tokens():
    q, kc, vc, table, ctx = _inputs(ctx=(9, 6, 13), n_q=1, bs=4)
    nb = kc.shape[0]
    t2 = table.clone()
    t2[0, 1] = -1          # tokens 4..7 of request 0
    t2[2, 0] = nb + 5      # tokens 0..3 of request 2
    o, lse = paged_decode_ref(q, kc, vc, t2, ctx)
    for b, drop in ((0, range(4, 8)), (2, range(0, 4))):
        n = int(ctx[b])
        keep = [t for t in range(n) if t not in drop]
        for h in range(4):
            k = _contiguous(kc, table[b], n, h // 2)[keep]
            v = _contiguous(vc, table[b], n, h // 2)[keep]
            s = (q[b, h, 0].double().numpy() @ k.T) / math.sqrt(16)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(o[b, h, 0], p @ v / p.sum(), atol=1e-12)
    o_ok, _ = paged_decode_ref(q, kc, vc, table, ctx)
    np.testing.assert_array_equal(o[1], o_ok[1])


def test_context_lengths_are_clamped():
    q, kc, vc, table, ctx = _inputs(ctx=(9, 4, 13), n_q=2, bs=4)
    o, lse = paged_decode_ref(q, kc, vc, table, ctx)
    # longer than max_ctx: only the first max_ctx tokens exist
    o2, lse2 = paged_decode_ref(q, kc, vc, table, torch.tensor([9, 4, 13]), max_ctx=9)
    o3, lse3 = paged_decode_ref(q, kc, vc, table, torch.tensor([9, 4, 9]))
    np.testing.assert_array_equal(o2, o3)
    np.testing.assert_array_equal(lse2, lse3)
    np.testing.assert_array_equal(o2[:2], o[:2])
    # longer than the block table holds: clamped to max_blocks * bs
    wide = torch.tensor([9, 4, 10 ** 6])
    o4, _ = paged_decode_ref(q, kc, vc, table, wide)
    o5, _ = paged_decode_ref(q, kc, vc, table,
                             torch.tensor([9, 4, table.shape[1] * 4]))
    np.testing.assert_array_equal(o4, o5)
    # nothing cached, and fewer cached tokens than query rows
    o6, lse6 = paged_decode_ref(q, kc, vc, table, torch.tensor([0, -3, 1]))
    assert np.all(o6[:2] == 0) and np.all(lse6[:2] == -np.inf)
    assert np.all(o6[2, :, 0] == 0) and np.all(lse6[2, :, 0] == -np.inf)
    assert np.all(np.isfinite(lse6[2, :, 1]))


# -- the seeded generator ---------------------------------------------------

def test_decode_generator_recipe():
    w = DECODE_WORKLOADS["decode_small"]
    q, kc, vc, table, ctx = generate_decode(w)
    assert ctx.tolist() == w.ctx_lens().tolist()
    need = [blocks_needed(int(n), w.block_size) for n in ctx]
    assert kc.shape == (sum(need) + w.extra_blocks, w.Hkv, w.block_size, w.d)
    owned = [int(e) for b in range(w.B) for e in table[b, :need[b]]]
    assert len(owned) == len(set(owned)) == sum(need)
    assert all(int(e) == -1 for b in range(w.B) for e in table[b, need[b]:])
    again = generate_decode(w)
    for x, y in zip((q, kc, vc, table, ctx), again):
        assert torch.equal(x, y)


def test_decode_workload_accounting():
    w = DECODE_WORKLOADS["decode_gqa_nq4"]
    ctx = [5, 1000]
    # row i of a request with n tokens sees n - n_q + i + 1 tokens
    per = sum(5 - 4 + i + 1 for i in range(4)) + sum(1000 - 4 + i + 1 for i in range(4))
    assert w.visible_pairs(ctx) == per * w.H
    assert w.compulsory_bytes(ctx) == 1005 * 2 * w.Hkv * w.d * 2 + \
        2 * w.B * w.H * 4 * w.d * 2 + 4 * w.B * w.H * 4

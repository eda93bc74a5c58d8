"""Host-side checks of the seeded input recipe and the work accounting."""
import numpy as np
import pytest
import torch

from oracle import visible
from workloads import WORKLOADS, input_digest, make_inputs


def test_inputs_are_deterministic_and_rounded_rne():
    a = make_inputs(1, 2, 64, 16, "bf16", seed=7)
    b = make_inputs(1, 2, 64, 16, "bf16", seed=7)
    assert input_digest(*a) == input_digest(*b)
    c = make_inputs(1, 2, 64, 16, "bf16", seed=8)
    assert input_digest(*a) != input_digest(*c)
    # draw order Q, K, V from one PCG64 stream, then RNE rounding
    rng = np.random.Generator(np.random.PCG64(7))
    qx = rng.standard_normal((1, 2, 64, 16), dtype=np.float32)
    kx = rng.standard_normal((1, 2, 64, 16), dtype=np.float32)
    assert torch.equal(a[0], torch.from_numpy(qx).to(torch.bfloat16))
    assert torch.equal(a[1], torch.from_numpy(kx).to(torch.bfloat16))
    assert all(t.is_contiguous() and t.dtype == torch.bfloat16 for t in a)


def test_outlier_rows_are_exactly_times_eight():
    plain = make_inputs(2, 2, 300, 8, "bf16", seed=3)
    out = make_inputs(2, 2, 300, 8, "bf16", seed=3, outliers=True)
    assert torch.equal(plain[0], out[0]) and torch.equal(plain[2], out[2])
    k0, k1 = plain[1].float(), out[1].float()
    changed = (k0 != k1).any(-1)
    assert changed.sum(-1).tolist() == [[3, 3], [3, 3]]
    assert torch.equal(k1[changed], 8 * k0[changed])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_visible_pairs_match_brute_count(name):
    w = WORKLOADS[name]
    S = min(w.S, 700)
    W = min(w.window, S // 3) if w.mask == "window" else None
    small = type(w)(**{**w.__dict__, "S": S, "window": W or 0, "B": 1, "H": 1})
    want = visible(np.arange(S), np.arange(S), w.mask, W).sum()
    assert small.visible_pairs() == want


def test_headline_work_figures():
    w = WORKLOADS["prefill_8k_d128"]
    assert w.visible_pairs() == 32 * 8192 * 8193 // 2
    assert abs(w.flops() - 5.498e11) / 5.498e11 < 1e-3
    assert abs(WORKLOADS["window_18k_d128"].flops() - 5.498e11) / 5.498e11 < 1e-3
    assert abs(WORKLOADS["full_d256_f16"].flops() - 1.100e12) / 1.1e12 < 1e-3
    assert abs(WORKLOADS["causal_d64"].flops() - 2.150e9) / 2.15e9 < 1e-3
    assert WORKLOADS["tiny_f32"].flops() == 4 * 64 * 2 * 256 * 256


def test_grouped_heads_generator_shapes_and_mha_identity():
    q, k, v = make_inputs(2, 8, 40, 16, "bf16", seed=9, Hkv=2)
    assert q.shape == (2, 8, 40, 16) and k.shape == v.shape == (2, 2, 40, 16)
    # Hkv == H draws exactly the plain multi-head inputs
    a = make_inputs(1, 4, 33, 8, "f16", seed=4)
    b = make_inputs(1, 4, 33, 8, "f16", seed=4, Hkv=4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_grouped_workload_counts():
    w = WORKLOADS["prefill_8k_d128_gqa4"]
    m = WORKLOADS["prefill_8k_d128"]
    assert w.kv_heads == 8 and m.kv_heads == 32
    assert w.flops() == m.flops()
    # Q and O are the same; K and V shrink by the group size (4)
    esz = 2
    assert m.compulsory_bytes() - w.compulsory_bytes() == 2 * (32 - 8) * 8192 * 128 * esz

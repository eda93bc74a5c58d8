"""GPU parity of the backward pass: the HIP kernels' dQ, dK, dV against the
fp64 oracle's exact gradients on identical seeded inputs.

Bar: every element within the first-order error bound of 16-bit storage with
fp32 accumulation (tests/bwd_bounds.py derives it; tests/test_bwd_bounds.py
shows that 16-bit rounding stays inside it and that plausible mistakes do
not).  The forward output and logsumexp fed to the backward are the HIP
forward's, as a caller would pass them.
"""
import math
import sys

import numpy as np
import pytest
import torch

import io_aware_tiled_flash_amd as fa
from bwd_bounds import excess, grad_bounds
from workloads import make_grad, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device (run with -m 'not gpu' on a host)")


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(B, H, Hkv, S, d, dtype, seed):
    q, k, v = make_inputs(B, H, S, d, dtype, seed, Hkv=Hkv)
    do = make_grad(B, H, S, d, dtype, seed + 7919)
    return q, k, v, do


def _run(q, k, v, do, mask, window, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, mask=mask, window=window, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, mask=mask, window=window, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _check(B, H, Hkv, S, d, dtype, mask, window=None, seed=11, scale=None):
    label = f"bwd {dtype} d={d} {mask} w={window} B={B} H={H} Hkv={Hkv} S={S} seed={seed}"
    _say(label)
    q, k, v, do = _inputs(B, H, Hkv, S, d, dtype, seed)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    got = _run(q, k, v, do, mask, window, scale)
    ref, bnd = grad_bounds(q, k, v, do, mask, window, scale, dtype)
    report = []
    for name, g, r, b in zip(("dq", "dk", "dv"), got, ref, bnd):
        assert torch.isfinite(g.float()).all(), f"{label}: {name} not finite"
        x = excess(g, r, b)
        report.append((name, x, _worst(g, r, b)))
    _say("  " + "  ".join(f"{n}: {x:.3f} of bound" for n, x, _ in report))
    for name, x, where in report:
        assert x <= 1.0, f"{label}: {name} error reaches {x:.3f} of its bound at {where}"
    return got


def _worst(got, ref, bound):
    err = np.abs(got.double().numpy() - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / bound)
    i = np.unravel_index(np.nanargmax(r), r.shape)
    return (f"index {tuple(int(t) for t in i)}: got {float(got[i]):.6g} "
            f"exact {ref[i]:.6g} bound {bound[i]:.3g}")


CASES = [
    # dtype, d, mask, H, Hkv, S, window
    ("bf16", 128, "causal", 2, 2, 256, None),   # whole tiles
    ("bf16", 128, "causal", 2, 2, 300, None),   # ragged tail
    ("bf16", 64, "causal", 2, 2, 300, None),
    ("bf16", 128, "none", 2, 2, 200, None),
    ("bf16", 64, "none", 1, 1, 333, None),
    ("f16", 128, "none", 1, 1, 333, None),
    ("f16", 64, "causal", 2, 2, 129, None),
    ("f16", 128, "causal", 1, 1, 511, None),
    ("bf16", 128, "window", 2, 2, 700, 100),
    ("bf16", 64, "window", 1, 1, 513, 33),
    ("f16", 128, "window", 1, 1, 400, 1),       # window of one: the diagonal only
    ("bf16", 128, "causal", 8, 2, 300, None),   # grouped heads
    ("f16", 64, "none", 6, 3, 257, None),
    ("bf16", 128, "causal", 4, 1, 200, None),   # one shared key/value head
    ("bf16", 128, "window", 4, 2, 333, 50),
    # unmasked with a multiple of 8 key/value heads: tiles of a head run in a
    # row on one XCD (the other unmasked cases keep the plain order)
    ("bf16", 128, "none", 8, 8, 300, None),
    ("f16", 64, "none", 16, 8, 200, None),
    # d = 256: wave pairs, each wave owning half of d for dK and dV
    ("bf16", 256, "causal", 2, 2, 300, None),
    ("f16", 256, "none", 1, 1, 200, None),
    ("bf16", 256, "window", 4, 2, 333, 70),
    ("f16", 256, "causal", 4, 1, 129, None),
]


@pytest.mark.parametrize("dtype,d,mask,H,Hkv,S,window", CASES)
def test_backward_full(dtype, d, mask, H, Hkv, S, window):
    _check(1, H, Hkv, S, d, dtype, mask, window)


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 127, 128, 129])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("d", [128, 256])
def test_backward_short_sequences(S, mask, d):
    # at d = 256: one or two 64-key work-groups, keys and rows past S zero-filled
    _check(1, 2, 2, S, d, "bf16", mask)


@pytest.mark.parametrize("d", [64, 256])
def test_backward_batch(d):
    _check(3, 2, 1, 190, d, "bf16", "causal")


@pytest.mark.parametrize("window", [1, 63, 64, 65])
def test_backward_d256_window_edges(window):
    """Windows around the 64-key work-group and 32-key wave-pair widths."""
    _check(1, 2, 1, 250, 256, "f16", "window", window)


@pytest.mark.parametrize("scale", [0.02, 1.0, -0.1])
def test_backward_scale_values(scale):
    _check(1, 1, 1, 160, 64, "bf16", "causal", scale=scale)


def test_backward_window_covering_sequence_is_causal_bitwise():
    q, k, v, do = _inputs(1, 2, 2, 300, 128, "bf16", 3)
    a = _run(q, k, v, do, "causal", None, 0.1)
    b = _run(q, k, v, do, "window", 300, 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [128, 256])
def test_backward_deterministic_repeat(d):
    q, k, v, do = _inputs(1, 4, 2, 400, d, "bf16", 4)
    a = _run(q, k, v, do, "causal", None, 0.09)
    b = _run(q, k, v, do, "causal", None, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 256])
def test_backward_outputs_do_not_touch_neighbours(d):
    """dq, dk, dv, delta carved out of larger buffers: the guard bytes around
    each stay untouched (at d = 256 each dK/dV work-group writes half of
    every row)."""
    _say(f"bwd guard bands d={d}")
    B, H, Hkv, S = 1, 2, 1, 200
    q, k, v, do = _inputs(B, H, Hkv, S, d, "bf16", 5)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, mask="causal")
    pad = 4096
    sizes = [B * H * S * d, B * Hkv * S * d, B * Hkv * S * d]
    bufs = [torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device=dev) for n in sizes]
    dl = torch.full((B * H * S + 2 * pad,), 3.0, dtype=torch.float32, device=dev)
    ptr = [b.data_ptr() + 2 * pad for b in bufs]
    st = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   dod.data_ptr(), ptr[0], ptr[1], ptr[2], dl.data_ptr() + 4 * pad, B, H, Hkv,
                   S, d, fa.DTYPES["bf16"], fa.MASKS["causal"], 0, 1.0 / math.sqrt(d),
                   torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    for b, n in zip(bufs, sizes):
        assert torch.all(b[:pad] == 7.0) and torch.all(b[pad + n:] == 7.0)
    assert torch.all(dl[:pad] == 3.0) and torch.all(dl[pad + B * H * S:] == 3.0)
    ref = fa.backward(qd, kd, vd, o, lse, dod, mask="causal")
    for b, n, r in zip(bufs, sizes, ref):
        assert torch.equal(b[pad:pad + n].view_as(r), r)


def _full_size(name):
    """One bench backward configuration at full size, run once on the GPU
    (inputs and gradients returned on the host)."""
    from workloads import WORKLOADS

    w = WORKLOADS[name]
    _say(f"bwd full-size {w.name}: launching")
    q, k, v = make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)
    do = make_grad(w.B, w.H, w.S, w.d, w.dtype, w.seed + 7919)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, mask=w.mask, window=w.window or None, scale=w.scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, mask=w.mask, window=w.window or None,
                             scale=w.scale)
    torch.cuda.synchronize()
    return w, (q, k, v, do), (dq.cpu(), dk.cpu(), dv.cpu()), lse.cpu()


@pytest.fixture(scope="module")
def full_size_backward():
    """The headline shape's backward (prefill_8k_d128) at full size."""
    return _full_size("prefill_8k_d128")


@pytest.fixture(scope="module")
def full_size_backward_d256():
    """The d = 256 backward workload (full_d256_f16: the wave-pair dK/dV
    kernel) at full size."""
    return _full_size("full_d256_f16")


def _identity(full):
    """Every head: sum_j dV[j] = sum_i dO[i] (each row's probabilities sum to
    one), within the sum of the per-element bounds, which for this identity
    needs only dO and dV."""
    from bwd_bounds import UNIT, F32

    w, (q, k, v, do), (dq, dk, dv), lse = full
    for name_, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(t.float()).all(), f"{name_} not finite"
    u = UNIT[w.dtype]
    g = (w.S + w.d + 16) * F32
    group = w.H // w.kv_heads
    qn = q.double().norm(dim=-1).amax().item()
    kn = k.double().norm(dim=-1).amax().item()
    rho = g * (abs(w.scale) * qn * kn + 1.0 + lse.abs().max().item() + 1e-3) + 4 * F32
    do64, dv64 = do.double(), dv.double()
    for b in range(w.B):
        for gh in range(w.kv_heads):
            heads = slice(gh * group, (gh + 1) * group)
            lhs = dv64[b, gh].sum(dim=0)
            rhs = do64[b, heads].sum(dim=(0, 1))
            tol = (u + g + rho) * do64[b, heads].abs().sum(dim=(0, 1)) \
                + u * dv64[b, gh].abs().sum(dim=0)
            gap = ((lhs - rhs).abs() / tol).max().item()
            assert gap <= 1.0, (f"batch {b} kv head {gh}: sum_j dV - sum_i dO reaches "
                                f"{gap:.3f} of bound")


def _every_element(full, pairs):
    """The (batch, head) slices in pairs: every element of dQ, dK and dV
    against the oracle's exact gradients, within its bound.  The slices run
    on a thread pool (the oracle's numpy work releases the GIL)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from bwd_bounds import UNIT, head_bounds
    from oracle import attention_bwd_rows_ref

    w, (q, k, v, do), (dq, dk, dv), _ = full
    assert w.kv_heads == w.H, "the whole-head check assumes one query head per kv head"
    u = UNIT[w.dtype]

    def one(bh):
        b, h = bh
        args = (q[b, h], k[b, h], v[b, h], do[b, h], w.mask, w.window or None, w.scale)
        ref = attention_bwd_rows_ref(*args)
        bnd = head_bounds(*args, w.dtype)
        out = []
        for got, r, e in zip((dq[b, h], dk[b, h], dv[b, h]), ref, bnd):
            out.append(excess(got, r, e + u * np.abs(r)))
        return out

    _say(f"bwd full-size {w.name}: (batch, head) {pairs[0]}..{pairs[-1]}, exact gradients "
         f"and bounds")
    workers = max(1, min(8, os.cpu_count() or 1))
    with threadpool_limits(limits=2), ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(one, pairs))
    for bh, xs in zip(pairs, res):
        _say(f"  {bh}: dq {xs[0]:.3f}, dk {xs[1]:.3f}, dv {xs[2]:.3f} of bound")
        for name_, x in zip(("dq", "dk", "dv"), xs):
            assert x <= 1.0, f"{bh}: {name_} error reaches {x:.3f} of its bound"


def test_backward_full_size_identity(full_size_backward):
    _identity(full_size_backward)


@pytest.mark.parametrize("first", [0, 8, 16, 24])
def test_backward_full_size_every_element(full_size_backward, first):
    """Heads first .. first+7 of the headline shape (B = 1, 32 heads)."""
    w = full_size_backward[0]
    _every_element(full_size_backward, [(0, h) for h in range(first, min(first + 8, w.H))])


def test_backward_d256_full_size_identity(full_size_backward_d256):
    _identity(full_size_backward_d256)


@pytest.mark.parametrize("first", [0, 16, 32, 48])
def test_backward_d256_full_size_every_element(full_size_backward_d256, first):
    """(batch, head) slices first .. first+15 of the 64 of the d = 256
    workload (B = 4, H = 16)."""
    w = full_size_backward_d256[0]
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)][first:first + 16]
    _every_element(full_size_backward_d256, pairs)

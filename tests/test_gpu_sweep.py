"""Seeded random sweep over the configuration space of all three entry points
(forward, backward, paged decode), each case against the fp64 oracle with
the same bars as the dedicated parity tests.  The cases are drawn once, from
a fixed seed, at collection time: the list is the same on every run.
"""
import math
import sys

import numpy as np
import pytest
import torch

import io_aware_tiled_flash_amd as fa
from bwd_bounds import excess, grad_bounds
from oracle import attention_ref, paged_decode_ref
from workloads import make_decode_inputs, make_grad, make_inputs

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device (run with -m 'not gpu' on a host)")


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _heads(rng):
    Hkv = int(rng.choice([1, 2, 3]))
    return Hkv * int(rng.choice([1, 2, 4])), Hkv


def _fwd_cases(n=16):
    rng = np.random.default_rng(7001)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.35, 0.2]))
        d = int(rng.choice([64, 128] if dtype == "f32" else [64, 128, 256]))
        mask = str(rng.choice(["none", "causal", "window"]))
        S = int(rng.integers(1, 700))
        H, Hkv = _heads(rng)
        B = int(rng.integers(1, 3))
        window = int(rng.integers(1, S + 40)) if mask == "window" else None
        out.append((i, dtype, d, mask, window, B, H, Hkv, S))
    return out


def _bwd_cases(n=12):
    rng = np.random.default_rng(7002)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "f16"]))
        d = int(rng.choice([64, 128]))
        mask = str(rng.choice(["none", "causal", "window"]))
        S = int(rng.integers(1, 400))
        H, Hkv = _heads(rng)
        B = int(rng.integers(1, 3))
        window = int(rng.integers(1, S + 40)) if mask == "window" else None
        out.append((i, dtype, d, mask, window, B, H, Hkv, S))
    return out


def _dec_cases(n=14):
    rng = np.random.default_rng(7003)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "f16"]))
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.choice([1, 2, 3, 4, 8, 16]))
        n_q = int(rng.choice([1, 1, 2, 3]))
        bs = int(rng.choice([1, 4, 16, 32, 128]))
        B = int(rng.integers(1, 5))
        hi = int(rng.choice([40, 600, 3000, 9000]))
        ctx = [int(x) for x in rng.integers(0, hi + 1, size=B)]
        out.append((i, dtype, d, B, H, Hkv, n_q, bs, tuple(ctx)))
    return out


@pytest.mark.parametrize("i,dtype,d,mask,window,B,H,Hkv,S", _fwd_cases())
def test_sweep_forward(i, dtype, d, mask, window, B, H, Hkv, S):
    _say(f"sweep fwd #{i}: {dtype} d={d} {mask} w={window} B={B} H={H} Hkv={Hkv} S={S}")
    q, k, v = make_inputs(B, H, S, d, dtype, 8000 + i, Hkv=Hkv)
    dev = torch.device("cuda:0")
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), mask=mask, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_ref(q, k, v, mask, window)
    do = np.abs(o.cpu().double().numpy() - o_ref).max()
    dl = np.abs(lse.cpu().double().numpy() - lse_ref).max()
    assert do <= O_TOL[dtype], f"max|dO| = {do}"
    assert dl <= LSE_TOL, f"max|dLSE| = {dl}"


@pytest.mark.parametrize("i,dtype,d,mask,window,B,H,Hkv,S", _bwd_cases())
def test_sweep_backward(i, dtype, d, mask, window, B, H, Hkv, S):
    _say(f"sweep bwd #{i}: {dtype} d={d} {mask} w={window} B={B} H={H} Hkv={Hkv} S={S}")
    q, k, v = make_inputs(B, H, S, d, dtype, 8100 + i, Hkv=Hkv)
    g = make_grad(B, H, S, d, dtype, 8200 + i)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, mask=mask, window=window)
    got = fa.backward(qd, kd, vd, o, lse, gd, mask=mask, window=window)
    torch.cuda.synchronize()
    ref, bnd = grad_bounds(q, k, v, g, mask, window, 1.0 / math.sqrt(d), dtype)
    for name, x, r, b in zip(("dq", "dk", "dv"), got, ref, bnd):
        e = excess(x.cpu(), r, b)
        assert e <= 1.0, f"{name} error reaches {e:.3f} of its bound"


@pytest.mark.parametrize("i,dtype,d,B,H,Hkv,n_q,bs,ctx", _dec_cases())
def test_sweep_decode(i, dtype, d, B, H, Hkv, n_q, bs, ctx):
    _say(f"sweep decode #{i}: {dtype} d={d} B={B} H={H} Hkv={Hkv} n_q={n_q} bs={bs} ctx={ctx}")
    q, kc, vc, table, c = make_decode_inputs(B, H, Hkv, n_q, d, dtype, bs, 8300 + i,
                                             ctx_lens=list(ctx), extra_blocks=3)
    max_ctx = max(max(ctx), 0)
    dev = torch.device("cuda:0")
    o, lse = fa.decode(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), c.to(dev),
                       max_ctx=max_ctx)
    torch.cuda.synchronize()
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, table, c, max_ctx=max_ctx)
    o64, l64 = o.cpu().double().numpy(), lse.cpu().double().numpy()
    empty = np.isneginf(lse_ref)
    assert np.all(np.isneginf(l64[empty])) and np.all(o64[empty] == 0)
    full = ~empty
    if full.any():
        assert np.abs(o64[full] - o_ref[full]).max() <= O_TOL[dtype]
        assert np.abs(l64[full] - lse_ref[full]).max() <= LSE_TOL

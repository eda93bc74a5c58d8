"""GPU parity: the HIP kernels against the fp64 oracle on identical seeded inputs.

Bars (stated for this path): max |O_gpu - O_oracle| <= 2e-2 for bf16 inputs,
5e-3 for fp16, 1e-5 for fp32; max |LSE_gpu - LSE_oracle| <= 1e-3.  Every
shape, the full-size workloads included (launched exactly as the benchmark
launches them), is compared element by element against the oracle over all
rows of all heads.  The full-size workloads also get a fast pre-check on
sampled rows and properties that hold at any size.
"""
import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import io_aware_tiled_flash_amd as fa
from oracle import attention_ref, attention_rows_ref
from workloads import WORKLOADS, make_inputs

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


def _run(q, k, v, mask, window, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, mask=mask, window=window, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_full(q, k, v, mask, window, scale, dtype, label):
    _say(label)
    o, lse = _run(q, k, v, mask, window, scale)
    o_ref, lse_ref = attention_ref(q, k, v, mask, window, scale)
    do = np.abs(o.double().numpy() - o_ref).max()
    dl = np.abs(lse.double().numpy() - lse_ref).max()
    assert do <= O_TOL[dtype], f"{label}: max|dO| = {do}"
    assert dl <= LSE_TOL, f"{label}: max|dLSE| = {dl}"
    return o, lse


def _sample_rows(S, n, rng):
    edge = [0, 1, 2, 31, 32, 63, 64, 127, 128, S // 2, S - 2, S - 1]
    rows = set(r for r in edge if 0 <= r < S)
    rows.update(rng.choice(S, min(n, S), replace=False).tolist())
    return np.array(sorted(rows))


def _check_sampled(q, k, v, o, lse, mask, window, scale, dtype, label, n_rows=48, seed=0):
    rng = np.random.default_rng(seed)
    B, H, S, d = q.shape
    group = H // k.shape[1]  # query heads per key/value head
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            rows = _sample_rows(S, n_rows, rng)
            g = h // group
            o_ref, lse_ref = attention_rows_ref(q[b, h], k[b, g], v[b, g], rows, mask, window,
                                                scale)
            worst_o = max(worst_o, np.abs(o[b, h, rows].double().numpy() - o_ref).max())
            worst_l = max(worst_l, np.abs(lse[b, h, rows].double().numpy() - lse_ref).max())
    assert worst_o <= O_TOL[dtype], f"{label}: sampled max|dO| = {worst_o}"
    assert worst_l <= LSE_TOL, f"{label}: sampled max|dLSE| = {worst_l}"


def _oracle_workers():
    # the oracle's elementwise numpy work releases the GIL on large arrays, so
    # a thread pool spreads the chunks over the host's cores (16 at most: the
    # share of one GPU's host)
    return max(1, min(16, os.cpu_count() or 1))


def _check_all_rows(q, k, v, o, lse, mask, window, scale, dtype, label, row_chunk=2048):
    """Every row of every head against the oracle, chunk by chunk (each
    chunk's scores and probabilities materialised in fp64, as attention_ref
    does), without holding the whole fp64 result."""
    from threadpoolctl import threadpool_limits

    B, H, S, d = q.shape
    group = H // k.shape[1]
    jobs = [(b, h, r0) for b in range(B) for h in range(H) for r0 in range(0, S, row_chunk)]

    def one(job):
        b, h, r0 = job
        rows = np.arange(r0, min(S, r0 + row_chunk))
        g = h // group
        o_ref, lse_ref = attention_rows_ref(q[b, h], k[b, g], v[b, g], rows, mask, window, scale)
        eo = float(np.abs(o[b, h, rows].double().numpy() - o_ref).max())
        el = float(np.abs(lse[b, h, rows].double().numpy() - lse_ref).max())
        return eo, el

    with threadpool_limits(limits=1), ThreadPoolExecutor(_oracle_workers()) as ex:
        res = list(ex.map(one, jobs))
    worst_o = max(r[0] for r in res)
    worst_l = max(r[1] for r in res)
    _say(f"{label}: all {B * H * S} rows, max|dO| = {worst_o:.3e}, max|dLSE| = {worst_l:.3e}")
    assert worst_o <= O_TOL[dtype], f"{label}: max|dO| = {worst_o}"
    assert worst_l <= LSE_TOL, f"{label}: max|dLSE| = {worst_l}"


# --------------------------------------------------------------------------
# the pages' worked example, through the kernel
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_worked_example_padded(dtype):
    """q = [1, 0] over four keys in two tiles (aicomputerinstitute.com flash-
    attention chapter, worked example), zero-padded to d = 64 and repeated
    over 4 query rows; every value is a small integer, exact in all dtypes."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    q = torch.zeros(1, 1, 4, 64, dtype=tdt)
    q[..., 0] = 1
    k = torch.zeros(1, 1, 4, 64, dtype=tdt)
    k[0, 0, :, :2] = torch.tensor([[1, 0], [0, 1], [3, 1], [-1, 1]], dtype=tdt)
    v = torch.zeros(1, 1, 4, 64, dtype=tdt)
    v[0, 0, :, :2] = torch.tensor([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=tdt)
    _say(f"worked example {dtype}")
    o, lse = _run(q, k, v, "none", None, 1.0)
    want = np.array([4.49786861, 5.49786861])
    tol = O_TOL[dtype]
    for i in range(4):
        assert np.abs(o[0, 0, i, :2].double().numpy() - want).max() <= tol
        assert float(o[0, 0, i, 2:].abs().max()) == 0.0
        assert abs(float(lse[0, 0, i]) - (3.0 + math.log(1.2034379904932108))) <= LSE_TOL


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "causal_d64", "causal_d64_outliers"])
def test_small_workloads_full(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)
    _check_full(q, k, v, w.mask, w.window or None, w.scale, w.dtype, name)


@pytest.mark.parametrize("name", ["prefill_8k_d128", "window_18k_d128", "full_d256_f16",
                                  "prefill_8k_d128_gqa4"])
def test_large_workloads_sampled(name):
    w = WORKLOADS[name]
    _say(f"{name}: generating inputs")
    q, k, v = make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)
    _say(f"{name}: launching")
    o, lse = _run(q, k, v, w.mask, w.window or None, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    # |O| is a convex combination of V rows, so it never exceeds max |V|
    assert float(o.float().abs().max()) <= float(v.float().abs().max()) * (1 + 1e-2)
    if w.mask != "none":  # causal/window row 0 sees only key 0 (of its key/value head)
        group = w.H // w.kv_heads
        k0 = torch.repeat_interleave(k[:, :, 0], group, dim=1)
        v0 = torch.repeat_interleave(v[:, :, 0], group, dim=1)
        s00 = (q[:, :, 0].double() * k0.double()).sum(-1) * w.scale
        assert float((lse[:, :, 0].double() - s00).abs().max()) <= LSE_TOL
        assert float((o[:, :, 0].float() - v0.float()).abs().max()) == 0.0
    _say(f"{name}: oracle rows")
    _check_sampled(q, k, v, o, lse, w.mask, w.window or None, w.scale, w.dtype, name)


@pytest.mark.parametrize("name", ["prefill_8k_d128", "window_18k_d128", "full_d256_f16",
                                  "prefill_8k_d128_gqa4"])
def test_large_workloads_every_row(name):
    """The full-size workloads, every output element and every logsumexp
    against the oracle."""
    w = WORKLOADS[name]
    _say(f"{name}: generating inputs")
    q, k, v = make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)
    _say(f"{name}: launching")
    o, lse = _run(q, k, v, w.mask, w.window or None, w.scale)
    _say(f"{name}: oracle over every row ({_oracle_workers()} threads)")
    _check_all_rows(q, k, v, o, lse, w.mask, w.window or None, w.scale, w.dtype, name)


# --------------------------------------------------------------------------
# shapes, masks, ragged tails
# --------------------------------------------------------------------------

GRID = [(dt, d, m) for dt in ("bf16", "f16") for d in (64, 128, 256)
        for m in ("none", "causal", "window")]


@pytest.mark.parametrize("dtype,d,mask", GRID)
@pytest.mark.parametrize("S", [1, 100, 257])
def test_grid_full(dtype, d, mask, S):
    window = 37 if mask == "window" else None
    q, k, v = make_inputs(1, 3, S, d, dtype, seed=S * 7 + d)
    _check_full(q, k, v, mask, window, 1.0 / math.sqrt(d), dtype,
                f"grid {dtype} d={d} {mask} S={S}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
@pytest.mark.parametrize("S", [1, 77, 300, 1500])
def test_f32_full(d, mask, S):
    window = 20 if mask == "window" else None
    q, k, v = make_inputs(2, 1, S, d, "f32", seed=S + d)
    _check_full(q, k, v, mask, window, 1.0 / math.sqrt(d), "f32", f"f32 d={d} {mask} S={S}")


@pytest.mark.parametrize("S,mask,window", [(1000, "causal", None), (4097, "none", None),
                                           (4097, "window", 700), (2049, "causal", None)])
def test_ragged_lengths(S, mask, window):
    q, k, v = make_inputs(1, 2, S, 128, "bf16", seed=S)
    _check_full(q, k, v, mask, window, 1.0 / math.sqrt(128), "bf16", f"ragged S={S} {mask}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,mask,window", [(64, "none", None), (64, "causal", None),
                                           (64, "window", 256), (64, "window", 333),
                                           (128, "window", 512), (128, "causal", None)])
def test_key_split_long_bands(dtype, d, mask, window):
    # B = 1, H = 2: the plain grid is far below one work-group per compute
    # unit, so the keys of every work-group are split over key groups (4 at
    # d = 64, 2 at d = 128) with many tiles per group; windows a multiple of
    # the 32-key tile and not, and a ragged S.
    S = 2900
    name, _ = fa.fa_query_fwd(1, 2, 2, S, d, fa.DTYPES[dtype], fa.MASKS[mask], window or 0)
    assert name.endswith(f"keysplit{4 if d == 64 else 2}>"), name
    q, k, v = make_inputs(1, 2, S, d, dtype, seed=d * 11 + (window or 0))
    _check_full(q, k, v, mask, window, 1.0 / math.sqrt(d), dtype,
                f"key split {dtype} d={d} {mask} W={window} S={S}")


@pytest.mark.parametrize("d,mask,window", [(128, "causal", None), (128, "window", 100),
                                           (64, "causal", None), (64, "window", 65)])
def test_plain_grid_last_rows_past_the_sequence(d, mask, window):
    # 64 heads of S = 900: at least 256 work-groups, so no key split, and
    # the last work-group of each head (rows 768..1023, or 896..1023 for the
    # 128-row d = 128 window instance) has waves whose rows all lie past S
    # and a wave that straddles it.
    name, grid = fa.fa_query_fwd(1, 64, 64, 900, d, fa.DTYPES["bf16"], fa.MASKS[mask],
                                 window or 0)
    br = 128 if (d, mask) == (128, "window") else 256
    assert "keysplit" not in name and f"br{br}" in name and grid == 64 * (1024 // br), \
        (name, grid)
    q, k, v = make_inputs(1, 64, 900, d, "bf16", seed=900 + d)
    _check_full(q, k, v, mask, window, 1.0 / math.sqrt(d), "bf16",
                f"plain grid d={d} {mask} W={window} S=900 H=64")


@pytest.mark.parametrize("dtype,d,B,H,Hkv,S", [("bf16", 128, 2, 16, 16, 2100),
                                                 ("bf16", 128, 2, 16, 4, 2100),
                                                 ("f16", 256, 4, 8, 8, 1000),
                                                 ("bf16", 64, 1, 56, 56, 1100),
                                                 ("bf16", 128, 1, 36, 36, 2100)])
def test_unmasked_head_order(dtype, d, B, H, Hkv, S):
    # Unmasked launches of at least 256 work-groups (no key split) with several
    # query tiles per head: B * H a multiple of 8 takes the order that runs a
    # head's query tiles in a row on one XCD; B * H = 36 keeps the plain order.
    name, grid = fa.fa_query_fwd(B, H, Hkv, S, d, fa.DTYPES[dtype], fa.MASKS["none"], 0)
    assert "keysplit" not in name and grid >= 256, (name, grid)
    q, k, v = make_inputs(B, H, S, d, dtype, seed=S + H + d, Hkv=Hkv)
    _check_full(q, k, v, "none", None, 1.0 / math.sqrt(d), dtype,
                f"unmasked order {dtype} d={d} B={B} H={H} Hkv={Hkv} S={S}")


def test_many_heads_small_sequence():
    q, k, v = make_inputs(3, 40, 65, 64, "bf16", seed=5)
    _check_full(q, k, v, "causal", None, 0.125, "bf16", "B=3 H=40 S=65")


@pytest.mark.parametrize("scale", [0.01, 1.0, 4.0])
def test_scale_values(scale):
    q, k, v = make_inputs(1, 2, 300, 128, "f16", seed=11)
    _check_full(q, k, v, "causal", None, scale, "f16", f"scale={scale}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 64)])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
@pytest.mark.parametrize("scale", [-0.125, 0.0])
def test_negative_and_zero_scale(dtype, d, mask, scale):
    """A negative scale (the matrix-core kernels flip Q's sign bits) and a
    zero scale (run as a vanishing positive one): against the oracle, and
    for scale 0 against the closed form, O = the mean of the visible V rows
    and LSE = ln(number of visible keys)."""
    S, window = 300, (41 if mask == "window" else None)
    q, k, v = make_inputs(1, 2, S, d, dtype, seed=17 + d)
    o, lse = _check_full(q, k, v, mask, window, scale, dtype,
                         f"scale={scale} {dtype} d={d} {mask}")
    if scale == 0.0:
        i = np.arange(S)
        lo = np.zeros(S, dtype=np.int64) if mask != "window" else np.maximum(0, i - window + 1)
        hi = np.full(S, S) if mask == "none" else i + 1
        csum = np.concatenate([np.zeros((1, 2, 1, d)), np.cumsum(v.double().numpy(), axis=2)],
                              axis=2)
        mean = (csum[:, :, hi] - csum[:, :, lo]) / (hi - lo)[None, None, :, None]
        assert np.abs(o.double().numpy() - mean).max() <= O_TOL[dtype]
        assert np.abs(lse.double().numpy() - np.log(hi - lo)).max() <= LSE_TOL


@pytest.mark.parametrize("dtype,jump", [("bf16", 26.0), ("f16", 7.0)])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_offset_moves(dtype, jump, d, mask):
    """Scores that climb (and fall) in 32-key plateaus.  The kernel lets a
    row's unnormalised weights grow up to 2^32 (bf16 weights) or 2^8 (fp16)
    before it moves the row's offset; steps of 1.5 * jump (natural units)
    exceed that, steps of 0.5 * jump do not, and some steps go down, so rows
    move their offset and rescale their accumulator several times, with
    earlier keys still contributing."""
    S = 300
    q, k, v = make_inputs(1, 2, S, d, dtype, seed=40 + d)
    scale = 1.0 / math.sqrt(d)
    blk = np.arange(S) // 32
    level = jump * (blk % 5) - 0.5 * jump * (blk % 2)
    q[..., 0] = 1.0
    k[..., 0] = torch.tensor(level / scale, dtype=torch.float32).to(k.dtype)
    _check_full(q, k, v, mask, 50 if mask == "window" else None, scale, dtype,
                f"offset moves {dtype} d={d} {mask}")


# --------------------------------------------------------------------------
# special cases with closed forms
# --------------------------------------------------------------------------

def test_zero_keys_average_visible_values():
    S = 200
    q, k, v = make_inputs(1, 2, S, 128, "bf16", seed=12)
    k = torch.zeros_like(k)
    _say("zero keys")
    o, lse = _run(q, k, v, "causal", None, 0.088)
    cum = torch.cumsum(v.double(), dim=2) / torch.arange(1, S + 1, dtype=torch.float64)[:, None]
    assert float((o.double() - cum).abs().max()) <= O_TOL["bf16"]
    want = torch.log(torch.arange(1, S + 1, dtype=torch.float64))
    assert float((lse.double() - want).abs().max()) <= LSE_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_window_of_one_returns_values(dtype):
    d = 64
    q, k, v = make_inputs(1, 2, 150, d, dtype, seed=13)
    _say(f"window=1 {dtype}")
    o, lse = _run(q, k, v, "window", 1, 0.125)
    assert torch.equal(o, v)
    s = (q.double() * k.double()).sum(-1) * 0.125
    assert float((lse.double() - s).abs().max()) <= LSE_TOL


def test_window_covering_sequence_is_causal_bitwise():
    q, k, v = make_inputs(1, 2, 333, 128, "bf16", seed=14)
    _say("window >= S")
    oc, lc = _run(q, k, v, "causal", None, 0.088)
    for W in (333, 334, 10_000):
        ow, lw = _run(q, k, v, "window", W, 0.088)
        assert torch.equal(ow, oc) and torch.equal(lw, lc)


def test_window_one_less_than_sequence():
    q, k, v = make_inputs(1, 2, 333, 128, "bf16", seed=15)
    _check_full(q, k, v, "window", 332, 0.088, "bf16", "window S-1")


def test_deterministic_repeat():
    w = WORKLOADS["causal_d64_outliers"]
    q, k, v = make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)
    _say("determinism")
    runs = [_run(q, k, v, "causal", None, w.scale) for _ in range(3)]
    for o, lse in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(lse, runs[0][1])


@pytest.mark.parametrize("dtype,d,B,H,Hkv,S,mask,window", [
    ("bf16", 128, 1, 32, 32, 2048, "causal", None),   # plain 256-row instance
    ("bf16", 128, 1, 16, 16, 3000, "window", 700),    # two-wave window instance
    ("f16", 256, 2, 16, 16, 1024, "none", None),      # d = 256, head-grouped order
    ("bf16", 128, 2, 16, 4, 1500, "none", None),      # grouped key/value heads
    ("f32", 128, 1, 8, 8, 700, "causal", None),       # fp32 quad-per-row kernel
])
def test_deterministic_repeat_instances(dtype, d, B, H, Hkv, S, mask, window):
    # Run-to-run bit identity of every instance family: no atomics, fixed
    # reduction orders.
    q, k, v = make_inputs(B, H, S, d, dtype, seed=S + d, Hkv=Hkv)
    _say(f"determinism {dtype} d={d} {mask} H={H} Hkv={Hkv} S={S}")
    runs = [_run(q, k, v, mask, window, 1.0 / math.sqrt(d)) for _ in range(3)]
    for o, lse in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(lse, runs[0][1])


@pytest.mark.parametrize("dtype,d,H,S,mask,window", [
    ("bf16", 64, 2, 130, "causal", None),     # key-split instance
    ("bf16", 128, 128, 300, "window", 70),    # plain two-wave window instance
    ("f16", 256, 64, 200, "none", None),      # d = 256, head-grouped order
    ("f32", 128, 4, 77, "window", 20),        # fp32 quad-per-row kernel
])
def test_outputs_do_not_touch_neighbours(dtype, d, H, S, mask, window):
    """The kernel writes exactly o and lse: guard bands around them stay intact."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(1, H, S, d, dtype, seed=16))
    n, nl = q.numel(), H * S
    big = torch.full((3 * n,), 7.0, dtype=q.dtype, device=dev)
    out = big[n:2 * n].view_as(q)
    lbig = torch.full((3 * nl,), 9.0, dtype=torch.float32, device=dev)
    lse = lbig[nl:2 * nl].view(1, H, S)
    _say(f"guard bands {dtype} d={d} H={H} S={S} {mask}")
    fa.forward(q, k, v, mask=mask, window=window, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((big[:n] == 7.0).all()) and bool((big[2 * n:] == 7.0).all())
    assert bool((lbig[:nl] == 9.0).all()) and bool((lbig[2 * nl:] == 9.0).all())
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())


def test_forward_refuses_host_outputs(monkeypatch):
    """out and lse must be device tensors on q's device: a host buffer would
    pass the library's pointer checks and fault in the kernel's stores.  The
    launch entry points are replaced by stubs that fail the test if called,
    so no kernel can run even if the check regressed."""
    def boom(*a, **kw):
        raise AssertionError("a kernel was launched with a host output buffer")

    monkeypatch.setattr(fa, "fa_fwd", boom)
    monkeypatch.setattr(fa, "fa_fwd_gqa", boom)
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device=dev)
    kg = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device=dev)
    o_host = torch.empty(1, 2, 64, 64, dtype=torch.bfloat16)
    l_host = torch.empty(1, 2, 64)
    o_dev = torch.empty_like(q)
    l_dev = torch.empty(1, 2, 64, device=dev)
    for kk in (q, kg):  # plain and grouped heads
        for out, lse in ((o_host, l_dev), (o_dev, l_host), (o_host, l_host)):
            with pytest.raises(fa.FaError) as e:
                fa.forward(q, kk, kk, mask="causal", out=out, lse=lse)
            assert e.value.status == fa.FA_EINVAL and "device" in str(e.value)


# --------------------------------------------------------------------------
# grouped key/value heads (fa_fwd_gqa): query head h uses key/value head
# h // (H / Hkv)
# --------------------------------------------------------------------------

GQA_CASES = [("bf16", 128, "causal", 8, 2, 300), ("bf16", 64, "none", 6, 3, 257),
             ("f16", 128, "window", 4, 1, 333), ("f16", 256, "causal", 4, 2, 130),
             ("bf16", 128, "none", 16, 8, 65), ("f32", 64, "causal", 4, 2, 100),
             ("f32", 128, "none", 3, 1, 77)]


@pytest.mark.parametrize("dtype,d,mask,H,Hkv,S", GQA_CASES)
def test_grouped_heads_full(dtype, d, mask, H, Hkv, S):
    window = 37 if mask == "window" else None
    q, k, v = make_inputs(2, H, S, d, dtype, seed=H * 100 + Hkv * 10 + d, Hkv=Hkv)
    _check_full(q, k, v, mask, window, 1.0 / math.sqrt(d), dtype,
                f"gqa {dtype} d={d} {mask} H={H} Hkv={Hkv} S={S}")


def test_grouped_heads_equal_repeated_heads_bitwise():
    # Grouping is exactly plain attention on repeated key/value heads: the
    # kernel must produce the same bits either way.
    q, k, v = make_inputs(1, 8, 200, 128, "bf16", seed=21, Hkv=2)
    dev = torch.device("cuda:0")
    _say("gqa vs repeated heads, bitwise")
    og, lg = fa.forward(q.to(dev), k.to(dev), v.to(dev), mask="causal")
    kr = torch.repeat_interleave(k, 4, dim=1).contiguous()
    vr = torch.repeat_interleave(v, 4, dim=1).contiguous()
    om, lm = fa.forward(q.to(dev), kr.to(dev), vr.to(dev), mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(og.cpu(), om.cpu())
    assert torch.equal(lg.cpu(), lm.cpu())

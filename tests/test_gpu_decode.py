"""GPU parity of paged-cache decoding: the HIP kernels against the fp64
oracle (oracle/decode.py) on identical seeded inputs.  Key/value heads that
serve up to 4 query rows run on the vector-ALU kernel, 5 or more on the
matrix-core kernel; the cases cover both, with and without split contexts.

Bars: the attention output bars, max |O_gpu - O_oracle| <= 2e-2 for bf16 and
5e-3 for fp16, max |LSE_gpu - LSE_oracle| <= 1e-3; rows with no visible
token must be exactly O = 0, LSE = -inf.  The full-size workloads are
launched exactly as the benchmark launches them and compared on every
request, head and row.
"""
import math
import sys

import numpy as np
import pytest
import torch

import io_aware_tiled_flash_amd as fa
from oracle import paged_decode_ref
from workloads import DECODE_WORKLOADS, generate_decode, make_decode_inputs

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 2e-2, "f16": 5e-3}
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device (run with -m 'not gpu' on a host)")


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(q, kc, vc, table, ctx, max_ctx, scale=None):
    dev = torch.device("cuda:0")
    o, lse = fa.decode(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), ctx.to(dev),
                       max_ctx=max_ctx, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _compare(o, lse, o_ref, lse_ref, dtype, label, rows=None):
    o64, l64 = o.double().numpy(), lse.double().numpy()
    if rows is not None:
        o64, l64, o_ref, lse_ref = o64[rows], l64[rows], o_ref[rows], lse_ref[rows]
    empty = np.isneginf(lse_ref)
    assert np.all(np.isneginf(l64[empty])), f"{label}: empty rows must have LSE = -inf"
    assert np.all(o64[empty] == 0), f"{label}: empty rows must have O = 0"
    full = ~empty
    assert np.all(np.isfinite(l64[full])), f"{label}: non-finite LSE"
    do = np.abs(o64[full] - o_ref[full]).max() if full.any() else 0.0
    dl = np.abs(l64[full] - lse_ref[full]).max() if full.any() else 0.0
    _say(f"  {label}: max|dO| {do:.2e}  max|dLSE| {dl:.2e}")
    assert do <= O_TOL[dtype], f"{label}: max|dO| = {do}"
    assert dl <= LSE_TOL, f"{label}: max|dLSE| = {dl}"


def _check(B, H, Hkv, n_q, d, dtype, bs, ctx, seed=21, extra=7, max_ctx=None, scale=None,
           table_edit=None):
    label = (f"decode {dtype} d={d} B={B} H={H} Hkv={Hkv} n_q={n_q} bs={bs} ctx={list(ctx)[:6]}"
             f"{'...' if len(ctx) > 6 else ''} max_ctx={max_ctx} seed={seed}")
    _say(label)
    q, kc, vc, table, ctxt = make_decode_inputs(B, H, Hkv, n_q, d, dtype, bs, seed,
                                                ctx_lens=list(ctx), extra_blocks=extra)
    if table_edit is not None:
        table = table_edit(table, kc.shape[0])
    if max_ctx is None:
        max_ctx = max(max(ctx), 0)
    o, lse = _run(q, kc, vc, table, ctxt, max_ctx, scale)
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, table, ctxt, max_ctx=max_ctx, scale=scale)
    _compare(o, lse, o_ref, lse_ref, dtype, label)
    return o, lse


CASES = [
    # dtype, d, B, H, Hkv, n_q, bs, ctx
    ("bf16", 128, 3, 4, 4, 1, 16, (1, 17, 300)),
    ("bf16", 128, 3, 8, 2, 1, 16, (5, 64, 1000)),
    ("f16", 128, 2, 8, 1, 1, 16, (33, 777)),
    ("bf16", 64, 4, 4, 2, 2, 16, (2, 16, 31, 129)),
    ("f16", 64, 2, 6, 3, 3, 8, (3, 250)),
    ("bf16", 128, 2, 4, 2, 1, 1, (7, 90)),          # one token per block
    ("bf16", 128, 2, 4, 2, 2, 64, (65, 200)),
    ("f16", 128, 1, 2, 2, 1, 1024, (1500,)),
    ("bf16", 128, 2, 32, 2, 1, 16, (40, 600)),       # 16 rows per key/value head: 2 slices
    ("bf16", 64, 1, 16, 2, 3, 16, (500,)),           # 24 rows: 3 slices
    ("bf16", 128, 1, 8, 8, 4, 16, (2,)),             # fewer cached tokens than query rows
    ("bf16", 128, 1, 64, 1, 1, 16, (700,)),          # 64 rows: two 32-row slices
    ("bf16", 128, 2, 2, 2, 1, 16, (5000, 3)),        # one row, split context
    ("f16", 64, 2, 4, 2, 1, 16, (4500, 33)),         # two rows, split context
    ("f16", 128, 2, 12, 4, 1, 32, (3000, 17)),       # three rows
    ("bf16", 128, 2, 16, 2, 2, 16, (3000, 40)),      # 16 rows, split context (matrix core)
    ("f16", 64, 3, 12, 1, 1, 16, (1, 129, 2500)),    # 12 rows (matrix core)
    ("bf16", 128, 2, 40, 4, 1, 16, (900, 5000)),     # 10 rows (matrix core)
    ("bf16", 128, 2, 28, 4, 1, 16, (900, 5000)),     # 7 rows (matrix core)
    ("bf16", 128, 2, 20, 4, 1, 16, (900, 5000)),     # 5 rows (matrix core)
    ("f16", 128, 2, 16, 4, 1, 16, (700, 4500)),      # 4 rows: vector
    ("f16", 64, 2, 16, 2, 1, 16, (3, 2100)),         # 8 rows (matrix core)
]


D256_CASES = [
    # dtype, d, B, H, Hkv, n_q, bs, ctx  (d = 256: 32 lanes per token)
    ("bf16", 256, 3, 4, 4, 1, 16, (1, 37, 700)),      # one row per key/value head
    ("f16", 256, 2, 4, 2, 1, 16, (5, 300)),           # two rows
    ("bf16", 256, 2, 8, 2, 1, 16, (64, 1000)),        # four rows
    ("f16", 256, 1, 16, 2, 2, 16, (900,)),            # 16 rows: four 4-row slices
    ("bf16", 256, 2, 8, 2, 1, 16, (5000, 33)),        # split context and merge
    ("bf16", 256, 1, 4, 1, 3, 8, (2500,)),            # 12 rows, split, n_q = 3
]


@pytest.mark.parametrize("dtype,d,B,H,Hkv,n_q,bs,ctx", D256_CASES)
def test_decode_head_dim_256(dtype, d, B, H, Hkv, n_q, bs, ctx):
    _check(B, H, Hkv, n_q, d, dtype, bs, ctx)


@pytest.mark.parametrize("dtype,d,B,H,Hkv,n_q,bs,ctx", CASES)
def test_decode_cases(dtype, d, B, H, Hkv, n_q, bs, ctx):
    _check(B, H, Hkv, n_q, d, dtype, bs, ctx)


@pytest.mark.parametrize("H", [8, 16])  # 4 rows per key/value head (vector kernel), 8 (matrix core)
def test_decode_more_than_64_splits(H):
    # A 70,000-token request in 1,024-token splits: the merge takes the
    # logsumexps of splits 64 and up from memory rather than from the wave's
    # lanes, and combines its partial rows in several groups.
    ws = fa.fa_decode_workspace_size(1, H, 2, 1, 128, 1, 16, 4400, 70000, 2)
    n_splits = ws // (H * 129 * 4)
    assert n_splits > 64, n_splits
    _check(1, H, 2, 1, 128, "bf16", 16, (70000,))


@pytest.mark.parametrize("ctx", [(5000,), (4096, 1, 12000), (9000, 0, 4097)])
def test_decode_long_contexts_are_split_and_merged(ctx):
    B = len(ctx)
    ws = fa.fa_decode_workspace_size(B, 8, 2, 1, 128, 1, 16, 1024, max(ctx), 2)
    assert ws > 0, "these sizes must take the split path"
    _check(B, 8, 2, 1, 128, "bf16", 16, ctx)


def test_decode_empty_and_clamped_contexts():
    # 0 and negative context lengths: empty rows; 700 > max_ctx 500: cut to 500
    q, kc, vc, table, _ = make_decode_inputs(4, 4, 2, 2, 128, "bf16", 16, 31,
                                             ctx_lens=[0, 5, 700, 1], extra_blocks=3)
    ctx = torch.tensor([0, -4, 700, 1], dtype=torch.int32)
    o, lse = _run(q, kc, vc, table, ctx, 500)
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, table, ctx, max_ctx=500)
    _compare(o, lse, o_ref, lse_ref, "bf16", "empty/clamped")
    assert np.all(np.isneginf(lse[:2].numpy()))


def test_decode_invalid_table_entries_hold_no_tokens():
    def edit(table, nb):
        t = table.clone()
        t[0, 1] = -1
        t[1, 0] = nb + 7
        t[1, 3] = -100
        t[2, :] = -1      # nothing valid at all
        return t
    _check(3, 4, 2, 2, 128, "bf16", 16, (60, 70, 40), table_edit=edit)


@pytest.mark.parametrize("scale", [0.01, 1.0, -0.2])
def test_decode_scale_values(scale):
    _check(2, 4, 2, 1, 64, "bf16", 16, (100, 333), scale=scale)


def test_decode_deterministic_repeat():
    q, kc, vc, table, ctx = make_decode_inputs(3, 8, 2, 2, 128, "bf16", 16, 41,
                                               ctx_lens=[3000, 20, 700], extra_blocks=2)
    a = _run(q, kc, vc, table, ctx, 3000)
    b = _run(q, kc, vc, table, ctx, 3000)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_outputs_do_not_touch_neighbours():
    B, H, Hkv, n_q, d, bs = 2, 4, 2, 1, 128, 16
    q, kc, vc, table, ctx = make_decode_inputs(B, H, Hkv, n_q, d, "bf16", bs, 43,
                                               ctx_lens=[5000, 30], extra_blocks=1)
    dev = torch.device("cuda:0")
    qd, kd, vd, td, cd = (t.to(dev) for t in (q, kc, vc, table, ctx))
    max_ctx = 5000
    nb, mb = kc.shape[0], table.shape[1]
    ws_bytes = fa.fa_decode_workspace_size(B, H, Hkv, n_q, d, nb, bs, mb, max_ctx, 2)
    assert ws_bytes > 0
    pad = 4096
    n_o = B * H * n_q * d
    ob = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device=dev)
    lb = torch.full((B * H * n_q + 2 * pad,), 3.0, dtype=torch.float32, device=dev)
    ws = torch.full((ws_bytes + 2 * pad,), 0x5a, dtype=torch.uint8, device=dev)
    st = fa.fa_decode_paged(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), td.data_ptr(),
                            cd.data_ptr(), ob.data_ptr() + 2 * pad, lb.data_ptr() + 4 * pad,
                            ws.data_ptr() + pad, ws_bytes, B, H, Hkv, n_q, d, nb, bs, mb,
                            max_ctx, 2, 1.0 / math.sqrt(d),
                            torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    assert torch.all(ob[:pad] == 7.0) and torch.all(ob[pad + n_o:] == 7.0)
    assert torch.all(lb[:pad] == 3.0) and torch.all(lb[pad + B * H * n_q:] == 3.0)
    assert torch.all(ws[:pad] == 0x5a) and torch.all(ws[pad + ws_bytes:] == 0x5a)
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, table, ctx, max_ctx=max_ctx)
    o = ob[pad:pad + n_o].view(B, H, n_q, d).cpu()
    lse = lb[pad:pad + B * H * n_q].view(B, H, n_q).cpu()
    _compare(o, lse, o_ref, lse_ref, "bf16", "guarded buffers")


@pytest.mark.parametrize("name", ["decode_small", "decode_opt13b_b256", "decode_gqa_long",
                                  "decode_gqa_nq4", "decode_gqa8", "decode_gqa_b256"])
def test_decode_workloads(name):
    """The named workloads at full size, launched as the benchmark launches
    them; every request, head and row against the oracle."""
    w = DECODE_WORKLOADS[name]
    _say(f"decode workload {name}")
    q, kc, vc, table, ctx = generate_decode(w)
    o, lse = _run(q, kc, vc, table, ctx, w.max_ctx, w.scale)
    assert torch.isfinite(o.float()).all()
    _say(f"decode workload {name}: oracle over all {w.B} requests")
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, table, ctx, max_ctx=w.max_ctx, scale=w.scale)
    _compare(o, lse, o_ref, lse_ref, w.dtype, f"{name} all requests")


# H, Hkv, n_q, ctx: 4 rows per key/value head (vector kernel) and 8 (matrix
# core); the long contexts take the split path.
SHARED_PREFIX_CASES = [(8, 2, 1, (700, 900, 650, 1200)), (16, 2, 1, (700, 900, 650, 1200)),
                       (8, 2, 1, (5000, 4100, 6000)), (8, 1, 2, (300, 2000, 520))]


@pytest.mark.parametrize("H,Hkv,n_q,ctx", SHARED_PREFIX_CASES)
def test_decode_shared_prefix_blocks(H, Hkv, n_q, ctx):
    """Copy-on-write prefix sharing (aicomputerinstitute.com flash-attention
    chapter, "PagedAttention: memory management borrowed from an operating
    system"): every request's table names request 0's physical blocks for its
    first P logical blocks.  Against the oracle, and bitwise against the same
    requests with the prefix copied into blocks of their own (the kernel
    reads through the table, so aliasing must not change a bit)."""
    B, d, bs, P = len(ctx), 128, 16, 18
    label = f"shared prefix H={H} Hkv={Hkv} n_q={n_q} ctx={ctx} P={P}"
    _say(label)
    q, kc, vc, table, ctxt = make_decode_inputs(B, H, Hkv, n_q, d, "bf16", bs, 77,
                                                ctx_lens=list(ctx), extra_blocks=4)
    shared = table.clone()
    kc_own, vc_own = kc.clone(), vc.clone()
    for b in range(1, B):
        shared[b, :P] = table[0, :P]
        kc_own[table[b, :P].long()] = kc[table[0, :P].long()]
        vc_own[table[b, :P].long()] = vc[table[0, :P].long()]
    max_ctx = max(ctx)
    o, lse = _run(q, kc, vc, shared, ctxt, max_ctx)
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, shared, ctxt, max_ctx=max_ctx)
    _compare(o, lse, o_ref, lse_ref, "bf16", label)
    o2, lse2 = _run(q, kc_own, vc_own, table, ctxt, max_ctx)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), f"{label}: aliasing changed bits"

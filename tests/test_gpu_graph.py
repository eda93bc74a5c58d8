"""The entry points inside a captured HIP graph.

fa_fwd, fa_bwd and fa_decode_paged allocate nothing and issue only kernel
launches on the caller's stream, so a caller may capture them (serving loops
replay captured graphs to skip per-launch host cost).  Each graph here holds
several calls of different instances; it is replayed several times with
other work on the GPU between replays, and every replay must reproduce the
eager results bit for bit.
"""
import math

import pytest
import torch

import io_aware_tiled_flash_amd as fa
from workloads import make_decode_inputs, make_grad, make_inputs

pytestmark = pytest.mark.gpu

CASES = [  # dtype, d, B, H, S, mask, window
    ("bf16", 64, 2, 8, 1024, "causal", None),    # key-split instance
    ("bf16", 128, 1, 32, 1000, "causal", None),  # plain instance, ragged S
    ("bf16", 128, 1, 16, 1500, "window", 300),   # two-wave window instance
    ("f16", 256, 2, 8, 600, "none", None),       # d = 256
    ("f32", 64, 1, 4, 300, "causal", None),      # fp32 kernel
]


def test_forward_calls_replay_bitwise_from_a_graph():
    dev = torch.device("cuda:0")
    calls = []
    for i, (dtype, d, B, H, S, mask, window) in enumerate(CASES):
        q, k, v = (t.to(dev) for t in make_inputs(B, H, S, d, dtype, seed=300 + i))
        out = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        calls.append((q, k, v, out, lse, mask, window, 1.0 / math.sqrt(d)))

    # eager reference results
    ref = []
    for q, k, v, _, _, mask, window, scale in calls:
        o, l = fa.forward(q, k, v, mask=mask, window=window, scale=scale)
        ref.append((o.clone(), l.clone()))
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for q, k, v, out, lse, mask, window, scale in calls:
            fa.forward(q, k, v, mask=mask, window=window, scale=scale, out=out, lse=lse,
                       stream=torch.cuda.current_stream(dev))
    torch.cuda.synchronize()

    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for _, _, _, out, lse, _, _, _ in calls:  # clear what the replay must rewrite
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
        junk = junk * 1.0001 + 1.0  # other work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, ((_, _, _, out, lse, _, _, _), (o_ref, l_ref)) in enumerate(zip(calls, ref)):
            assert torch.equal(out, o_ref), f"replay {rep}, case {CASES[i]}: O differs"
            assert torch.equal(lse, l_ref), f"replay {rep}, case {CASES[i]}: LSE differs"


def _bwd_call(dtype, d, B, H, Hkv, S, mask, window, seed, dev):
    """Preallocated buffers of one fa_bwd call and a closure that issues it."""
    q, k, v = (t.to(dev) for t in make_inputs(B, H, S, d, dtype, seed=seed, Hkv=Hkv))
    do = make_grad(B, H, S, d, dtype, seed + 1).to(dev)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, mask=mask, window=window, scale=scale)
    bufs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
            torch.empty((B, H, S), dtype=torch.float32, device=dev)]

    def issue(stream):
        st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       do.data_ptr(), *[t.data_ptr() for t in bufs], B, H, Hkv, S, d,
                       fa.DTYPES[dtype], fa.MASKS[mask], int(window or 0), scale,
                       stream.cuda_stream)
        assert st == fa.FA_OK, fa.fa_last_error()
    return bufs, issue


def _decode_call(dtype, d, B, H, Hkv, n_q, bs, ctx, seed, dev):
    """Preallocated buffers (workspace included) of one fa_decode_paged call
    and a closure that issues it."""
    q, kc, vc, table, ctxt = (t.to(dev) for t in make_decode_inputs(
        B, H, Hkv, n_q, d, dtype, bs, seed, ctx_lens=ctx, extra_blocks=3))
    max_ctx = max(ctx)
    nb, mb = kc.shape[0], table.shape[1]
    ws_bytes = fa.fa_decode_workspace_size(B, H, Hkv, n_q, d, nb, bs, mb, max_ctx,
                                           fa.DTYPES[dtype])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    bufs = [torch.empty_like(q), torch.empty((B, H, n_q), dtype=torch.float32, device=dev)]

    def issue(stream):
        st = fa.fa_decode_paged(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), table.data_ptr(),
                                ctxt.data_ptr(), bufs[0].data_ptr(), bufs[1].data_ptr(),
                                ws.data_ptr(), ws.numel(), B, H, Hkv, n_q, d, nb, bs, mb,
                                max_ctx, fa.DTYPES[dtype], 1.0 / math.sqrt(d),
                                stream.cuda_stream)
        assert st == fa.FA_OK, fa.fa_last_error()
    return bufs, issue


def test_backward_and_decode_calls_replay_bitwise_from_a_graph():
    """fa_bwd (three launches, the caller's row-term buffer) and
    fa_decode_paged (split and merge launches, the caller's workspace) also
    allocate nothing: captured together, every replay reproduces the eager
    results bit for bit."""
    dev = torch.device("cuda:0")
    calls = [
        _bwd_call("bf16", 128, 1, 8, 2, 700, "causal", None, 400, dev),  # grouped heads
        _bwd_call("f16", 256, 1, 4, 4, 300, "none", None, 401, dev),     # d = 256 wave pairs
        _bwd_call("bf16", 64, 2, 2, 2, 333, "window", 50, 402, dev),
        _decode_call("bf16", 128, 3, 8, 8, 1, 16, [5000, 37, 1200], 403, dev),  # split + merge
        _decode_call("f16", 128, 2, 32, 4, 4, 16, [900, 2049], 404, dev),  # matrix-core path
        _decode_call("bf16", 256, 2, 4, 2, 1, 32, [700, 3000], 405, dev),
    ]
    stream = torch.cuda.current_stream(dev)
    for _, issue in calls:
        issue(stream)
    torch.cuda.synchronize()
    ref = [[t.clone() for t in bufs] for bufs, _ in calls]

    cap = torch.cuda.Stream(device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for _, issue in calls:
            issue(cap)
    torch.cuda.synchronize()

    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for bufs, _ in calls:
            for t in bufs:
                t.fill_(float("nan") if t.is_floating_point() else 0)
        junk = junk * 1.0001 + 1.0
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, ((bufs, _), r) in enumerate(zip(calls, ref)):
            for j, (t, tr) in enumerate(zip(bufs, r)):
                assert torch.equal(t, tr), f"replay {rep}, call {i}, output {j} differs"

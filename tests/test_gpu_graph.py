"""The forward entry point inside a captured HIP graph.

fa_fwd allocates nothing and issues only its kernel launch on the caller's
stream, so a caller may capture it (serving loops replay captured graphs to
skip per-launch host cost).  Each graph here holds several forward calls of
different instances; it is replayed several times with other work on the GPU
between replays, and every replay must reproduce the eager results bit for
bit.
"""
import math

import pytest
import torch

import io_aware_tiled_flash_amd as fa
from workloads import make_inputs

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

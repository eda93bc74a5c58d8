"""fa_decode_paged_noalloc against fa_decode_paged through the C ABI.

(Named to be collected last: it must pass alone in a fresh process and after
every other GPU test.)

The allocation-free entry point runs the same kernels with the library's own
static split scratch in place of the caller's workspace, so its outputs must
equal fa_decode_paged's bit for bit (and both must meet the oracle's bars).
Two calls in a row, the second smaller than the first, show that what the
first call left in the scratch does not leak into the second.
"""
import math
import sys

import numpy as np
import pytest
import torch

import io_aware_tiled_flash_amd as fa
from oracle import paged_decode_ref
from workloads import make_decode_inputs

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


def _both(q, kc, vc, table, ctx, max_ctx, dtype):
    """(o, lse) of fa_decode_paged with a torch workspace, then of
    fa_decode_paged_noalloc, on the same device inputs."""
    dev = torch.device("cuda:0")
    qd, kd, vd, td, cd = (t.to(dev) for t in (q, kc, vc, table, ctx))
    B, H, n_q, d = q.shape
    nb, Hkv, bs, _ = kc.shape
    mb = table.shape[1]
    dt = fa.DTYPES[dtype]
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = fa.fa_decode_workspace_size(B, H, Hkv, n_q, d, nb, bs, mb, max_ctx, dt)
    assert 0 < ws_bytes <= fa.NOALLOC_SCRATCH_BYTES, "these cases must take the split path"
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o1, o2 = torch.empty_like(qd), torch.empty_like(qd)
    l1 = torch.empty((B, H, n_q), dtype=torch.float32, device=dev)
    l2 = torch.empty_like(l1)
    st = fa.fa_decode_paged(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), td.data_ptr(),
                            cd.data_ptr(), o1.data_ptr(), l1.data_ptr(), ws.data_ptr(),
                            ws_bytes, B, H, Hkv, n_q, d, nb, bs, mb, max_ctx, dt, scale, stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    st = fa.fa_decode_paged_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), td.data_ptr(),
                                    cd.data_ptr(), o2.data_ptr(), l2.data_ptr(), B, H, Hkv, n_q,
                                    d, nb, bs, mb, max_ctx, dt, scale, stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    return (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu())


def _case(B, H, Hkv, n_q, d, dtype, ctx, seed):
    label = f"noalloc decode {dtype} d={d} B={B} H={H} Hkv={Hkv} n_q={n_q} ctx={ctx}"
    _say(label)
    q, kc, vc, table, ctxt = make_decode_inputs(B, H, Hkv, n_q, d, dtype, 16, seed,
                                                ctx_lens=list(ctx), extra_blocks=3)
    (o1, l1), (o2, l2) = _both(q, kc, vc, table, ctxt, max(ctx), dtype)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{label}: differs from fa_decode_paged"
    o_ref, lse_ref = paged_decode_ref(q, kc, vc, table, ctxt, max_ctx=max(ctx))
    do = np.abs(o2.double().numpy() - o_ref).max()
    dl = np.abs(l2.double().numpy() - lse_ref).max()
    _say(f"  {label}: max|dO| {do:.2e} max|dLSE| {dl:.2e}")
    assert do <= O_TOL[dtype] and dl <= LSE_TOL, label


def test_noalloc_decode_matches_decode_twice_second_smaller():
    # first call: 4 rows per key/value head (vector kernel), long contexts,
    # many splits; second call: smaller, 8 rows per key/value head (matrix
    # cores), fewer splits over a smaller part of the scratch
    _case(4, 32, 8, 1, 128, "bf16", (9000, 20000, 3000, 12000), seed=91)
    _case(2, 16, 2, 1, 128, "bf16", (5000, 700), seed=92)


def test_noalloc_decode_fp16_d64_and_several_new_tokens():
    _case(3, 12, 4, 2, 64, "f16", (4100, 2, 6000), seed=93)
    _case(1, 4, 2, 1, 64, "f16", (3000,), seed=94)

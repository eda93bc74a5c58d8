"""Benchmark of the attention forward pass on one MI355X.

One step is one ``fa_fwd`` launch over the whole batch of the workload (all
of the hot path: tile loads, QK^T, masking, online softmax, PV, epilogue).
With ``--pass bwd`` a step is one ``fa_bwd`` call instead (gradients of the
same workload, given the forward's outputs and a seeded output gradient).
Inputs are generated once, copied to HBM and reused.  Before the W untimed
warm-up steps a clock-settling phase repeats the step for ``--settle-s``
seconds (default 1; 0 disables it): under sustained matrix-core load the
MI355X shader clock takes on the order of a second to settle, and a few
warm-up steps alone time it cold (about a quarter slower).  The phase is
declared in the output line (``clock_settle``).  Then K steps are timed with
events on the launch stream (one event between consecutive steps, so the
mean, median and minimum step times are all reported), bracketed by
synchronisation.  A shader-clock sample taken on the same stream right
before and right after the timed steps gives the mean clock over them, and
the line quotes the percentage of peak both against the published peak
(2.4 GHz) and against the peak at that measured clock.  After the timed steps
a matrix-core ceiling run (``mfma_ceiling``; ``--no-ceiling`` skips it)
measures what the MFMA units sustain on operands like the inputs with
nothing else to do, and the line also gives the kernel's fraction of that.

Prints one JSON line: the headline metric (forward TFLOP/s, causal FLOPs
counted as 4*d per visible pair) plus a ``roofline`` object for the kernel and
a ``cpu_baseline`` object (the fp64 oracle timed on a bounded sample of the
same workload on the host cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s at S=8K,d=128 bf16 causal; % of MFMA bf16 peak"
HEADLINE = "prefill_8k_d128"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # dense: MFMA bf16/f16, fp32 vector
PEAK_CLOCK_MHZ = 2400.0  # the clock the published peaks assume
HBM_PEAK_GBS = 8000.0
# Backward FLOPs: five products of 2*d FLOPs per visible (row, key) pair (S and
# dP recomputed once, dV, dK, dQ) against the forward's two, the usual
# accounting; recomputing S and dP a second time for dQ is not counted.
BWD_FLOP_RATIO = 2.5
# The backward's kernels issue 14*d FLOPs per visible pair (the dK/dV kernel
# recomputes S and dP, and so does the dQ kernel): 1.4 times the credited 10*d.
BWD_ISSUED_RATIO = 1.4
BWD_KERNELS = ("fa_bwd_delta_kernel", "fa_bwd_dkdv_kernel", "fa_bwd_dq_kernel")
GRAD_SEED_OFFSET = 7919  # dO is drawn with seed = the workload's seed + this
DECODE_DEFAULT = "decode_opt13b_b256"
CSRC = os.path.join(ROOT, "io_aware_tiled_flash_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# The sources each measured kernel is compiled from: a committed counter
# summary is only used while these are unchanged.
FWD_SOURCES = ("fa_fwd_mfma.hip", "fa_gfx950.h", "fa_internal.h")
DECODE_SOURCES = ("fa_decode.hip", "fa_tile_ops.h", "fa_gfx950.h", "fa_internal.h")
BWD_SOURCES = ("fa_bwd_mfma.hip", "fa_tile_ops.h", "fa_gfx950.h", "fa_internal.h")


def kernel_source_digest(sources=FWD_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sources=FWD_SOURCES):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; otherwise None."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, _, val = line.partition(":")
            vals[key.strip()] = val.strip()
    # (the digest line may name its sources after the digest)
    if (vals.get("kernel_source_digest") or "").split()[:1] != [kernel_source_digest(sources)]:
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def host_cpu() -> dict:
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, and the model name."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"host_cpus": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])


class ClockSampler:
    """Mean shader clock over a stretch of stream work, from the per-die
    cycle and real-time counters (libfa_clock.so, measurement support)."""

    N_WG = 1024  # work-groups per sample: almost every compute unit gets some

    def __init__(self, device, stream):
        import ctypes

        import torch
        path = os.path.join(ROOT, "io_aware_tiled_flash_amd", "libfa_clock.so")
        self.lib = ctypes.CDLL(path)
        self.lib.fa_clock_sample.restype = ctypes.c_int
        self.lib.fa_clock_sample.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        self.lib.fa_clock_realtime_khz.restype = ctypes.c_int
        self.real_khz = self.lib.fa_clock_realtime_khz()
        self.bufs = [torch.zeros(3 * self.N_WG, dtype=torch.int64, device=device)
                     for _ in range(2)]
        self.stream = stream

    def sample(self, i: int) -> None:
        st = self.lib.fa_clock_sample(self.bufs[i].data_ptr(), self.N_WG,
                                      self.stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"clock sample launch failed ({st})")

    def mean_mhz(self):
        """Mean clock (MHz) between samples 0 and 1: per compute unit seen in
        both samples (cycle counters of different units are not aligned),
        then the mean over units, and per die."""
        if self.real_khz <= 0:
            return None
        a, b = (x.cpu().view(-1, 3).tolist() for x in self.bufs)
        first, last = {}, {}
        for cu, cyc, real in a:
            first.setdefault(cu, (cyc, real))
        for cu, cyc, real in b:
            last.setdefault(cu, (cyc, real))
        per_cu = {}
        for cu in set(first) & set(last):
            dc = last[cu][0] - first[cu][0]
            dr = last[cu][1] - first[cu][1]
            if dr > 0 and dc > 0:
                per_cu[cu] = dc / (dr / (self.real_khz * 1e3)) / 1e6
        if not per_cu:
            return None
        dies = {}
        for cu, mhz in per_cu.items():
            dies.setdefault(cu & 0xF, []).append(mhz)
        vals = sorted(per_cu.values())
        return {"mean_MHz": round(sum(vals) / len(vals), 1),
                "median_MHz": round(vals[len(vals) // 2], 1),
                "min_MHz": round(vals[0], 1), "max_MHz": round(vals[-1], 1),
                "compute_units": len(vals),
                "per_die_MHz": {str(d_): round(sum(v_) / len(v_), 1)
                                for d_, v_ in sorted(dies.items())},
                "method": "per compute unit: shader-cycle counter over the real-time counter, "
                          "sampled on the launch stream right before and after the timed steps"}


def mfma_ceiling(device, stream, dtype: str, clock: "ClockSampler", launch_s: float = 0.25,
                 settle_s: float = 1.0):
    """Sustained matrix-core rate of this part on operands like the inputs
    (roughly standard normal bf16 or fp16), with nothing else in the loop
    (libfa_clock.so, measurement support): launches of 32 x 32 x 16 MFMA
    chains run for about settle_s, then two launches are timed between
    events, with a clock sample on either side.  Under sustained load the
    power limit sets the clock, so no kernel on such operands can beat this
    rate; the attention kernels are also quoted as a fraction of it."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "io_aware_tiled_flash_amd", "libfa_clock.so"))
    lib.fa_mfma_ceiling.restype = ctypes.c_int
    lib.fa_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint, ctypes.c_void_p]
    code = {"f16": 1, "bf16": 2}[dtype]
    n_wg = 8192  # 32 per compute unit: the tail of the last round is small
    out = torch.empty(256 * n_wg, dtype=torch.float32, device=device)

    def launch(rounds):
        st = lib.fa_mfma_ceiling(out.data_ptr(), n_wg, rounds, code, 12345, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"MFMA ceiling launch failed ({st})")

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        launch(64)
        ev[1].record(stream)
        stream.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        rounds = max(64, int(64 * launch_s * 1e3 / max(ms, 1e-3)))
        t0 = time.time()
        while time.time() - t0 < settle_s:
            launch(rounds)
            stream.synchronize()
        clock.sample(0)
        ev[0].record(stream)
        launch(rounds)
        launch(rounds)
        ev[1].record(stream)
        clock.sample(1)
        stream.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    flop = 2.0 * n_wg * 4 * rounds * 64 * 32768
    tflops = flop / (ms * 1e-3) / 1e12
    clk = clock.mean_mhz()
    return {"TFLOP/s": round(tflops, 1),
            "frac_of_published_peak": round(tflops / PEAK_TFLOPS[dtype], 4),
            "clock_MHz": clk["mean_MHz"] if clk else None,
            "seconds_timed": round(ms * 1e-3, 3), "settle_s": settle_s,
            "method": "v_mfma_f32_32x32x16 chains on register operands drawn about standard "
                      "normal, 4 independent accumulators per wave, no memory traffic"}


def time_steps(step, stream, steps: int, warmup: int, settle_s: float, clock=None):
    """Settle the clock, warm up, then time `steps` back-to-back calls between
    one pair of events (the mean step time, the figure the line reports), with
    a clock sample on either side.  A second, separately reported pass of the
    same number of steps puts an event between consecutive steps for the
    median, minimum and maximum (those events cost a few microseconds per
    step, which matters for short kernels, so they stay out of the mean).
    Returns (mean ms, per-step ms of the second pass, settle record)."""
    import torch
    settle = {"seconds": 0.0, "steps": 0}
    if settle_s > 0:
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < settle_s:
            for _ in range(10):
                step()
            n += 10
            torch.cuda.synchronize()
        settle = {"seconds": round(time.perf_counter() - t0, 3), "steps": n}
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if clock is not None:
        clock.sample(0)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    if clock is not None:
        clock.sample(1)
    torch.cuda.synchronize()
    mean_ms = start.elapsed_time(end) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return mean_ms, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)], settle


def time_graph(run, stream, steps: int, warmup: int, settle_s: float, clock=None):
    """Graph mode (forward only): settle and warm up with ordinary launches,
    then capture `steps` calls of run(stream) once into a HIP graph on a side
    stream and time one replay of it on `stream` between a pair of events.
    The host issues one launch for all the steps, so short kernels are timed
    back to back instead of at the host's launch rate.  Returns what
    time_steps does (every step taken as the mean)."""
    import torch
    settle = {"seconds": 0.0, "steps": 0}
    if settle_s > 0:
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < settle_s:
            for _ in range(10):
                run(stream)
            n += 10
            torch.cuda.synchronize()
        settle = {"seconds": round(time.perf_counter() - t0, 3), "steps": n}
    for _ in range(warmup):
        run(stream)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream(device=stream.device)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(steps):
            run(cap)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()  # untimed: the first replay uploads the graph
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if clock is not None:
            clock.sample(0)
        start.record(stream)
        graph.replay()
        end.record(stream)
        if clock is not None:
            clock.sample(1)
    torch.cuda.synchronize()
    mean_ms = start.elapsed_time(end) / steps
    return mean_ms, [mean_ms] * steps, settle


def step_stats(mean_ms, ms_list):
    srt = sorted(ms_list)
    n = len(srt)
    med = srt[n // 2] if n % 2 else 0.5 * (srt[n // 2 - 1] + srt[n // 2])
    return {"mean": round(mean_ms, 4),
            "per_step_pass": {"median": round(med, 4), "min": round(srt[0], 4),
                              "max": round(srt[-1], 4),
                              "note": "a second pass with an event between steps"}}


def cpu_baseline(w, q, k, v, target_s: float):
    """Time the fp64 oracle on whole heads of the workload's own (host) inputs
    until ~target_s of wall time has passed."""
    from oracle import attention_ref

    threads = blas_threads()
    per_head_pairs = w.visible_pairs() // (w.B * w.H)
    group = w.H // w.kv_heads
    t0 = time.perf_counter()
    heads = 0
    while True:
        b, h = divmod(heads, w.H)
        g = h // group
        attention_ref(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                      w.mask, w.window or None, w.scale)
        heads += 1
        el = time.perf_counter() - t0
        if el >= target_s or heads >= w.B * w.H:
            break
    flops = 4.0 * w.d * per_head_pairs * heads
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of {w.name} (all {w.S} query rows each, "
                      f"fp64 numpy, S and P materialised in 2048-row chunks), {el:.1f} s",
            "seconds": round(el, 2), "threads": "numpy BLAS threads (the elementwise steps "
                                                "run on one)", **host_cpu()}


def cpu_baseline_bwd(w, q, k, v, do, target_s: float):
    """Time the fp64 oracle's gradients on whole heads until ~target_s."""
    from oracle import attention_bwd_rows_ref

    threads = blas_threads()
    per_head_pairs = w.visible_pairs() // (w.B * w.H)
    group = w.H // w.kv_heads
    t0 = time.perf_counter()
    heads = 0
    while True:
        b, h = divmod(heads, w.H)
        g = h // group
        attention_bwd_rows_ref(q[b, h], k[b, g], v[b, g], do[b, h], w.mask, w.window or None,
                               w.scale)
        heads += 1
        el = time.perf_counter() - t0
        if el >= target_s or heads >= w.B * w.H:
            break
    flops = BWD_FLOP_RATIO * 4.0 * w.d * per_head_pairs * heads
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"gradients of {heads} of {w.B * w.H} heads of {w.name} (all {w.S} "
                      f"rows, fp64 numpy, P materialised per head), {el:.1f} s",
            "seconds": round(el, 2), "threads": "numpy BLAS threads (the elementwise steps "
                                                "run on one)", **host_cpu()}


def cpu_baseline_decode(w, q, kc, vc, table, ctx, target_s: float):
    """Time the fp64 oracle on whole requests until ~target_s; GB/s of the
    same byte accounting as the GPU figure, over the requests it finished."""
    from oracle import paged_decode_ref
    from workloads import kv_bytes_per_token

    threads = blas_threads()
    t0 = time.perf_counter()
    done = []
    while True:
        b = len(done)
        paged_decode_ref(q, kc, vc, table, ctx, max_ctx=w.max_ctx, scale=w.scale, requests=[b])
        done.append(b)
        el = time.perf_counter() - t0
        if el >= target_s or len(done) >= w.B:
            break
    c = ctx.numpy()[done]
    # the same accounting as DecodeWorkload.compulsory_bytes, for these requests
    byt = int(c.sum()) * kv_bytes_per_token(w.Hkv, w.d, w.esz) + \
        len(done) * w.H * w.n_q * (2 * w.d * w.esz + 4)
    return {"value": byt / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(done)} of {w.B} requests of {w.name} (every head and row; fp64 "
                      f"numpy gather + softmax), {el:.1f} s", "seconds": round(el, 2),
            "threads": "numpy BLAS threads (the elementwise steps run on one)", **host_cpu()}


def bench_decode(args) -> int:
    """One step = one fa_decode_paged call over the whole batch of requests."""
    import torch

    import io_aware_tiled_flash_amd as fa
    from workloads import DECODE_WORKLOADS, generate_decode

    name = args.workload if args.workload in DECODE_WORKLOADS else DECODE_DEFAULT
    w = DECODE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    host = generate_decode(w)
    q, kc, vc, table, ctx = (t.to(dev) for t in host)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.n_q), dtype=torch.float32, device=dev)
    nb, mb = kc.shape[0], table.shape[1]
    dt = fa.DTYPES[w.dtype]
    ws_bytes = fa.fa_decode_workspace_size(w.B, w.H, w.Hkv, w.n_q, w.d, nb, w.block_size, mb,
                                           w.max_ctx, dt)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = (q.data_ptr(), kc.data_ptr(), vc.data_ptr(), table.data_ptr(), ctx.data_ptr(),
            o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), w.B, w.H, w.Hkv, w.n_q,
            w.d, nb, w.block_size, mb, w.max_ctx, dt, float(w.scale), stream.cuda_stream)

    def step():
        st = fa.fa_decode_paged(*call)
        if st != fa.FA_OK:
            raise fa.FaError(st, fa.fa_last_error())

    warm = args.warmup
    clock = ClockSampler(dev, stream)
    mean_ms, times, settle = time_steps(step, stream, args.steps, warm, args.settle_s, clock)
    stats = step_stats(mean_ms, times)
    ms = mean_ms
    c = host[4].numpy()
    byt = w.compulsory_bytes(c)
    gbs = byt / (ms * 1e-3) / 1e9
    tflops = w.flops(c) / (ms * 1e-3) / 1e12
    result = {
        "metric": f"paged decode GB/s on {w.name} (cache rows read once + q, o, lse); "
                  f"% of HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "n_q": w.n_q,
                   "d": w.d, "block_size": w.block_size, "ctx": [w.ctx_lo, w.ctx_hi],
                   "cached_tokens": int(c.sum()), "pass": "decode",
                   "splits": "none" if ws_bytes == 0 else "split + merge",
                   "rows_per_kv_head": w.H // w.Hkv * w.n_q,
                   "kernel": "fa_decode_paged" + ("" if ws_bytes == 0 else " + merge")},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, DECODE_SOURCES),
                     "scope": "whole call (one launch without splits, two with)"},
        "attention_TFLOPs": round(tflops, 2),
        "step_ms": stats,
        "clock_settle": settle,
        "clock": clock.mean_mhz(),
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_decode(w, *host, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def copy_calibration(args) -> int:
    """Plain copy of a known byte count per step, for scaling HBM counters."""
    import torch
    n = args.copy_calibration_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(json.dumps({"copy_bytes_read_per_step": n, "copy_bytes_written_per_step": n,
                      "ms_per_step": round(ms, 4), "GBps": round(2 * n / ms / 1e6, 1)}),
          flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of repeated steps before the warm-up, so that the shader "
                         "clock reaches its loaded level (declared in the output; 0: none)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--graph", action="store_true",
                    help="forward only: capture the timed steps once in a HIP graph and time "
                         "one replay (short workloads are otherwise timed at the host's "
                         "launch rate)")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd", "decode"), default="fwd",
                    help="time the forward pass (the headline), the backward pass, or "
                         "paged-cache decoding (workload default: " + DECODE_DEFAULT + ")")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the matrix-core ceiling run (about 1.5 s) that the forward and "
                         "backward lines are also quoted against")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of attention, run a plain device-to-device copy of this "
                         "many MiB per step (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each head's work needs no exchange with another's, so a multi-GPU run "
              "would shard by batch and heads, one share per GPU). Run with --gpus 1.",
              file=sys.stderr)
        return 2
    if args.graph and args.pass_ != "fwd":
        print("--graph times the forward pass only", file=sys.stderr)
        return 2

    import torch

    import io_aware_tiled_flash_amd as fa
    from workloads import WORKLOADS, make_grad, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    if args.copy_calibration_mib > 0:
        return copy_calibration(args)
    if args.pass_ == "decode":
        return bench_decode(args)
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    host = make_inputs(w.B, w.H, w.S, w.d, w.dtype, w.seed, w.sigma, w.outliers, w.kv_heads)
    q, k, v = (t.to(dev) for t in host)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    window = w.window or None
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.forward(q, k, v, mask=w.mask, window=window, scale=w.scale, out=o, lse=lse,
                   stream=stream)

    if args.pass_ == "bwd":
        # the forward once (untimed) for O and the logsumexp, then the timed
        # step is one fa_bwd call (all three of its launches)
        step()
        dout = make_grad(w.B, w.H, w.S, w.d, w.dtype, w.seed + GRAD_SEED_OFFSET).to(dev)
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        delta = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
        bwd_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    delta.data_ptr(), w.B, w.H, w.kv_heads, w.S, w.d, fa.DTYPES[w.dtype],
                    fa.MASKS[w.mask], int(w.window or 0), float(w.scale), stream.cuda_stream)

        def step():  # noqa: F811
            st = fa.fa_bwd(*bwd_args)
            if st != fa.FA_OK:
                raise fa.FaError(st, fa.fa_last_error())

    clock = ClockSampler(dev, stream)
    if args.graph:
        def run(s):
            fa.forward(q, k, v, mask=w.mask, window=window, scale=w.scale, out=o, lse=lse,
                       stream=s)
        mean_ms, times, settle = time_graph(run, stream, args.steps, args.warmup,
                                            args.settle_s, clock)
        stats = {"mean": round(mean_ms, 4),
                 "note": "one graph replay of all the steps: no per-step times"}
    else:
        mean_ms, times, settle = time_steps(step, stream, args.steps, args.warmup,
                                            args.settle_s, clock)
        stats = step_stats(mean_ms, times)
    ms = mean_ms
    clk = clock.mean_mhz()

    bwd = args.pass_ == "bwd"
    flops = w.flops() * (BWD_FLOP_RATIO if bwd else 1.0)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    # the backward's traffic is that of its dominant launch, the dK/dV kernel
    traffic = (measured_traffic(f"{w.name}_bwd_dkdv", BWD_SOURCES) if bwd
               else measured_traffic(w.name))
    if bwd:
        metric = (f"attention bwd TFLOP/s on {w.name} (10*d FLOPs per visible pair); "
                  f"% of MFMA {w.dtype} peak")
        kernel = "fa_bwd: " + ", ".join(BWD_KERNELS)
    else:
        # fp32 inputs run on the vector ALUs (no down-conversion): their peak
        # is the fp32 vector rate, and the bound is the ALUs, not the MFMA
        unit_name = "fp32 vector" if w.dtype == "f32" else f"MFMA {w.dtype}"
        metric = METRIC if w.name == HEADLINE else (
            f"attention fwd TFLOP/s on {w.name}; % of {unit_name} peak")
        kernel = fa.fa_query_fwd(w.B, w.H, w.kv_heads, w.S, w.d, fa.DTYPES[w.dtype],
                                 fa.MASKS[w.mask], int(w.window or 0))[0]
    result = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "S": w.S,
                   "d": w.d,
                   "mask": w.mask, "window": w.window or None, "input_dtype": w.dtype,
                   "pass": args.pass_, "kernel": kernel},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "alu" if w.dtype == "f32" else "mfma",
                     "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic},
        "step_ms": stats,
        "launch": ("graph: the timed steps captured once, one replay timed" if args.graph
                   else "stream: one launch per step from the host"),
        "clock_settle": settle,
        "clock": clk,
        "hbm": {"compulsory_bytes": w.compulsory_bytes(),
                "compulsory_GBps": round(w.compulsory_bytes() / (ms * 1e-3) / 1e9, 1),
                "peak_GBps": HBM_PEAK_GBS},
    }
    if clk is not None:
        # the same peak rate per clock (256 CUs x 4096 flop/clk for bf16/fp16
        # MFMA) at the clock measured over the timed steps
        peak_at = peak * clk["mean_MHz"] / PEAK_CLOCK_MHZ
        result["pct_of_peak_at_measured_clock"] = round(100.0 * tflops / peak_at, 2)
        result["roofline"]["peak_at_measured_clock"] = round(peak_at, 1)
        result["roofline"]["frac_at_measured_clock"] = round(tflops / peak_at, 4)
    issued_ratio = 1.0
    if bwd:
        issued_ratio = BWD_ISSUED_RATIO
        result["roofline"]["scope"] = ("whole pass (three launches); traffic: HBM bytes of "
                                       "one dK/dV launch")
        result["roofline"]["mfma_flop_issued_per_credited"] = issued_ratio
    if args.ceiling and w.dtype in ("bf16", "f16"):
        ceil = mfma_ceiling(dev, stream, w.dtype, clock)
        result["mfma_ceiling"] = ceil
        issued = tflops * issued_ratio
        result["roofline"]["frac_of_mfma_ceiling"] = round(issued / ceil["TFLOP/s"], 4)
    if args.cpu_seconds > 0:
        if bwd:
            result["cpu_baseline"] = cpu_baseline_bwd(w, *host, dout.cpu(), args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline(w, *host, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

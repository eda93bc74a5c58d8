"""Measurement support: the clock/ceiling library's argument checks, the
profile summaries computed from small synthetic rocprofv3 outputs, and (on a
GPU) the clock sampler and the matrix-core ceiling run that bench.py quotes."""
import contextlib
import csv
import ctypes
import io
import os

import pytest

import bench
from io_aware_tiled_flash_amd import profsum

CLOCK_LIB = os.path.join(bench.ROOT, "io_aware_tiled_flash_amd", "libfa_clock.so")


def _clock_lib():
    lib = ctypes.CDLL(CLOCK_LIB)
    lib.fa_clock_sample.restype = ctypes.c_int
    lib.fa_clock_sample.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.fa_mfma_ceiling.restype = ctypes.c_int
    lib.fa_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint, ctypes.c_void_p]
    return lib


def test_clock_library_refuses_bad_arguments_before_any_launch():
    lib = _clock_lib()
    fake = 0x7F0000000000  # never dereferenced: every call below fails its checks first
    assert lib.fa_clock_sample(None, 16, None) == -1
    assert lib.fa_clock_sample(fake, 0, None) == -1
    assert lib.fa_clock_sample(fake, 4097, None) == -1
    assert lib.fa_clock_sample(fake + 4, 16, None) == -1  # not 8-byte aligned
    assert lib.fa_mfma_ceiling(None, 8, 1, 2, 1, None) == -1
    assert lib.fa_mfma_ceiling(fake, 0, 1, 2, 1, None) == -1
    assert lib.fa_mfma_ceiling(fake, 8, 0, 2, 1, None) == -1
    assert lib.fa_mfma_ceiling(fake, 8, 1, 0, 1, None) == -1  # fp32 has no such run
    assert lib.fa_mfma_ceiling(fake + 2, 8, 1, 1, 1, None) == -1


def test_bench_graph_mode_is_forward_only():
    # refused before anything touches a GPU
    assert bench.main(["--graph", "--pass", "bwd"]) == 2
    assert bench.main(["--graph", "--pass", "decode"]) == 2


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _run(argv):
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        assert profsum.main(argv) == 0
    return buf.getvalue()


def _value(text, key):
    for line in text.splitlines():
        if line.strip().startswith(key + ":"):
            return line.split(":", 1)[1].split()[0]
    raise KeyError(key)


def test_trace_summary_means_over_the_last_calls(tmp_path):
    # kernel A: durations 100, 200, 300, 400 ns; kernel B: one call of 50 ns
    rows, t = [], 1000
    for dur in (100, 200, 300, 400):
        rows.append(["A(args)", t, t + dur])
        t += 1000
    rows.append(["B(args)", t, t + 50])
    _write_csv(tmp_path / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp",
                                                   "End_Timestamp"], rows)
    out = _run(["trace", "--dir", str(tmp_path), "--workload", "prefill_8k_d128", "--last", "2",
                "--cmd", "the command"])
    a = out[out.index("kernel: A(args)"):out.index("kernel: B(args)")]
    assert "calls: 4" in a
    assert _value(a, "average_ns (all calls)") == "250"
    assert _value(a, "average_ns_last_2_calls (bench.py timed steps)") == "350"
    assert _value(a, "median_ns_last_2_calls") == "350"
    assert "#   the command" in out and "kernel_source_digest:" in out


COUNTER_HEADER = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"]


def test_sq_summary_derives_clock_busy_and_mfma_count(tmp_path):
    # one dispatch of 500 us; counters split over two per-die rows (summed)
    d = tmp_path / "sq"
    d.mkdir()
    dur = 500_000
    per_die = {
        "GRBM_GUI_ACTIVE": 8 * 2.0 * dur / 2,        # 2.0 GHz on each of 8 dies
        "SQ_WAVE_CYCLES": 4096 * 1_000_000 / 4 / 2,  # 4096 waves alive 1e6 cycles each
        "SQ_WAVES": 4096 / 2,
        "SQ_ACTIVE_INST_ANY": 4096 * 500_000 / 4 / 2,
        "SQ_VALU_MFMA_BUSY_CYCLES": 4096 * 600_000 / 2,
        "SQ_INSTS_MFMA": 5.498229e11 / 32768 / 2,
    }
    rows = []
    for half in range(2):
        for name, v in per_die.items():
            rows.append([7, "fa_fwd_mfma_kernel<x>", name, v, 10, 10 + dur])
    _write_csv(d / "p_counter_collection.csv", COUNTER_HEADER, rows)
    out = _run(["sq", "--dir", str(d), "--workload", "prefill_8k_d128", "--kernel",
                "fa_fwd_mfma", "--last", "1", "--cmd", "c"])
    assert float(_value(out, "clock_GHz (GRBM_GUI_ACTIVE / 8 dies / dispatch time)")) == \
        pytest.approx(2.0)
    assert float(_value(out, "issued / algorithmic")) == pytest.approx(1.0, abs=1e-3)
    assert _value(out, "issuing") == "50.0%"
    assert _value(out, "matrix core busy") == "60.0%"
    # 4096 waves x 1e6 cycles over 1024 SIMDs x 1e6 dispatch cycles = 4 waves per SIMD
    assert float(_value(out, "mean resident waves per SIMD over the dispatch")) == \
        pytest.approx(4.0)


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    dirs = {}
    for k in ("fetch", "write", "cfetch", "cwrite"):
        dirs[k] = tmp_path / k
        dirs[k].mkdir()
    kib = 256 * 1024  # the 256 MiB copy
    _write_csv(dirs["cfetch"] / "a_counter_collection.csv", COUNTER_HEADER,
               [[1, "copy_kernel", "FETCH_SIZE", kib / 2, 0, 1]])  # reads half the bytes
    _write_csv(dirs["cwrite"] / "a_counter_collection.csv", COUNTER_HEADER,
               [[1, "copy_kernel", "WRITE_SIZE", kib, 0, 1]])
    _write_csv(dirs["fetch"] / "a_counter_collection.csv", COUNTER_HEADER,
               [[3, "fa_fwd_mfma_kernel", "FETCH_SIZE", 1000.0, 0, 1],
                [4, "fa_fwd_mfma_kernel", "FETCH_SIZE", 3000.0, 0, 1],
                [5, "other", "FETCH_SIZE", 9e9, 0, 1]])
    _write_csv(dirs["write"] / "a_counter_collection.csv", COUNTER_HEADER,
               [[3, "fa_fwd_mfma_kernel", "WRITE_SIZE", 500.0, 0, 1]])
    out = _run(["traffic", "--fetch", str(dirs["fetch"]), "--write", str(dirs["write"]),
                "--copy-fetch", str(dirs["cfetch"]), "--copy-write", str(dirs["cwrite"]),
                "--workload", "prefill_8k_d128", "--kernel", "fa_fwd_mfma", "--cmd", "c"])
    assert float(_value(out, "fetch_scale")) == pytest.approx(2.0)
    assert float(_value(out, "hbm_read_bytes_per_launch")) == pytest.approx(2000 * 2 * 1024)
    assert float(_value(out, "hbm_write_bytes_per_launch")) == pytest.approx(500 * 1024)
    assert float(_value(out, "hbm_bytes_per_launch")) == pytest.approx(4500 * 1024)


@pytest.mark.gpu
def test_clock_sampler_and_mfma_ceiling_give_plausible_figures():
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    clock = bench.ClockSampler(dev, stream)
    # The shader-cycle counters only advance while the compute units work, so
    # the samples go around back-to-back launches (library set-up first).
    with torch.cuda.stream(stream):
        a = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
        b = a @ a
        stream.synchronize()
        clock.sample(0)
        for _ in range(200):
            b = a @ a
        clock.sample(1)
    stream.synchronize()
    clk = clock.mean_mhz()
    assert clk is not None and clk["compute_units"] >= 200, clk
    assert 300.0 < clk["min_MHz"] <= clk["max_MHz"] < 3000.0, clk
    ceil = bench.mfma_ceiling(dev, stream, "bf16", clock, launch_s=0.05, settle_s=0.1)
    assert 200.0 < ceil["TFLOP/s"] < 1.05 * bench.PEAK_TFLOPS["bf16"], ceil
    assert ceil["clock_MHz"] is not None and 300.0 < ceil["clock_MHz"] < 3000.0, ceil

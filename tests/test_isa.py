"""Checks of the generated gfx950 code (host only: the sources are compiled to
device assembly with the library's own flags; nothing runs on a GPU).

* M0 is written only by the kernels' inline direct-to-LDS loads, each
  `s_mov_b32 m0, <sgpr>` immediately followed by its `buffer_load ... lds`.
  The compiler treats M0 as reserved and ignores clobber lists naming it, so
  a compiler-generated use of M0 (an indexed register move, for instance)
  could silently read the value the asm left there; none may appear.
* No packed-fp32 arithmetic (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32)
  anywhere: every source is built with that target feature switched off.
* The forward, backward and decode kernels keep everything in registers and
  LDS (no scratch spills).
* In the backward's wave-pair dK/dV kernel every LDS write (the fp32 tiles
  the two waves of a pair exchange) is complete before the next barrier: on
  this part the compiler puts no wait in front of s_barrier, so the kernel
  waits by hand, and the partner's read after the barrier relies on it.
"""
import os
import re
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from io_aware_tiled_flash_amd import build as B

SOURCES = ["fa_fwd_mfma.hip", "fa_bwd_mfma.hip", "fa_decode.hip", "fa_fwd_f32.hip",
           "fa_clock.hip"]


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as td:
        outs = [os.path.join(td, s + ".s") for s in SOURCES]
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            list(ex.map(B.device_asm, SOURCES, outs))
        yield {s: open(o).read().splitlines() for s, o in zip(SOURCES, outs)}


def _code(lines):
    for i, line in enumerate(lines):
        t = line.split(";", 1)[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            yield i, t


@pytest.mark.parametrize("src", SOURCES)
def test_m0_only_feeds_the_direct_lds_loads(asm, src):
    code = list(_code(asm[src]))
    for k, (i, t) in enumerate(code):
        if not re.search(r"\bm0\b", t):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", t), f"{src}:{i + 1}: compiler use of m0: {t}"
        nxt = code[k + 1][1] if k + 1 < len(code) else ""
        assert re.match(r"buffer_load_dword(x4)? .* lds$", nxt), \
            f"{src}:{i + 1}: m0 set but not consumed by the next instruction ({nxt})"


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32_arithmetic(asm, src):
    bad = [t for _, t in _code(asm[src]) if re.match(r"v_pk_(add|mul|fma)_f32\b", t)]
    assert not bad, f"{src}: {bad[:3]}"


@pytest.mark.parametrize("src", ["fa_fwd_mfma.hip", "fa_bwd_mfma.hip", "fa_decode.hip",
                                 "fa_fwd_f32.hip"])
def test_no_scratch_spills(asm, src):
    sizes = [int(m.group(1)) for m in
             (re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", ln) for ln in asm[src]) if m]
    assert sizes and max(sizes) == 0, f"{src}: private segment sizes {sorted(set(sizes))}"


def _kernel_bodies(lines, name):
    """Code lines of each kernel whose symbol contains name."""
    bodies, cur = [], None
    for ln in lines:
        if re.match(r"^_Z\S*:", ln):
            cur = [] if name in ln else None
            if cur is not None:
                bodies.append(cur)
        elif cur is not None:
            if ln.strip().startswith(".end_amdhsa_kernel") or "s_endpgm" in ln:
                cur.append(ln)
                cur = None
            else:
                cur.append(ln)
    return bodies


def test_pair_kernel_lds_writes_complete_before_each_barrier(asm):
    bodies = _kernel_bodies(asm["fa_bwd_mfma.hip"], "fa_bwd_dkdv_pair_kernel")
    assert bodies, "no wave-pair dK/dV kernel in the backward's code"
    writes = 0
    for body in bodies:
        code = list(_code(body))
        for k, (i, t) in enumerate(code):
            if not t.startswith("ds_write"):
                continue
            writes += 1
            for _, u in code[k + 1:]:
                if u.startswith("s_waitcnt") and "lgkmcnt(0)" in u:
                    break
                assert not u.startswith("s_barrier"), \
                    f"LDS write at line {i + 1} ({t}) not awaited before a barrier"
    assert writes > 0

"""MI355X (gfx950) exact attention, forward and backward: Python binding of
``libfa.so``.

The functions ``fa_fwd``, ``fa_fwd_gqa``, ``fa_bwd``, ``fa_decode_paged``,
``fa_decode_paged_noalloc``, ``fa_decode_workspace_size``, ``fa_query``,
``fa_query_fwd``, ``fa_status_str``, ``fa_last_error`` and ``fa_abi_version``
mirror the C ABI declared in ``include/fa.h`` one to one (argument
marshalling only).  ``forward``, ``backward`` and ``decode`` are the
tensor-level convenience wrappers: they check the tensors, allocate the
outputs with torch and launch on torch's current stream.  Every arithmetic
step runs in the HIP kernels; there is no Python or CPU fallback, and a
missing library is an error.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FaError", "fa_fwd", "fa_fwd_gqa", "fa_bwd", "fa_decode_paged",
           "fa_decode_paged_noalloc", "fa_decode_workspace_size", "NOALLOC_SCRATCH_BYTES",
           "fa_query", "fa_query_fwd", "fa_status_str", "fa_last_error", "fa_abi_version",
           "forward", "backward", "decode", "library_path", "DTYPES", "MASKS", "FA_OK",
           "FA_EINVAL", "FA_EUNSUPPORTED", "FA_EHIP"]

FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_EHIP = 0, 1, 2, 3
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
MASKS = {"none": 0, "causal": 1, "window": 2}
ABI_VERSION = 1
NOALLOC_SCRATCH_BYTES = 16 << 20  # FA_NOALLOC_SCRATCH_BYTES

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfa.so"
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_text(status)}: {detail}" if detail else _status_text(status))


def library_path() -> str:
    """The in-tree libfa.so, or another build of the same sources named by
    the environment variable IO_AWARE_FA_LIBRARY (for instance one whose host
    code is compiled with AddressSanitizer)."""
    return os.environ.get("IO_AWARE_FA_LIBRARY") or os.path.join(_PKG, _LIB_NAME)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FaError(FA_EHIP, f"{path} is missing; build it with "
                               "`python -m io_aware_tiled_flash_amd.build`")
    lib = ctypes.CDLL(path)
    i64, c_int = ctypes.c_int64, ctypes.c_int
    lib.fa_fwd.restype = c_int
    lib.fa_fwd.argtypes = [ctypes.c_void_p] * 5 + [i64] * 4 + [c_int, c_int, i64,
                                                               ctypes.c_float, ctypes.c_void_p]
    lib.fa_fwd_gqa.restype = c_int
    lib.fa_fwd_gqa.argtypes = [ctypes.c_void_p] * 5 + [i64] * 5 + [c_int, c_int, i64,
                                                                   ctypes.c_float,
                                                                   ctypes.c_void_p]
    lib.fa_bwd.restype = c_int
    lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [i64] * 5 + [c_int, c_int, i64,
                                                                ctypes.c_float, ctypes.c_void_p]
    lib.fa_decode_paged.restype = c_int
    lib.fa_decode_paged.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_size_t] + [i64] * 9 +
                                    [c_int, ctypes.c_float, ctypes.c_void_p])
    lib.fa_decode_paged_noalloc.restype = c_int
    lib.fa_decode_paged_noalloc.argtypes = ([ctypes.c_void_p] * 7 + [i64] * 9 +
                                            [c_int, ctypes.c_float, ctypes.c_void_p])
    lib.fa_decode_workspace_size.restype = c_int
    lib.fa_decode_workspace_size.argtypes = [i64] * 9 + [c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_query.restype = c_int
    lib.fa_query.argtypes = [i64, c_int, c_int, ctypes.c_char_p, ctypes.c_size_t]
    lib.fa_query_fwd.restype = c_int
    lib.fa_query_fwd.argtypes = [i64] * 5 + [c_int, c_int, i64, ctypes.c_char_p,
                                             ctypes.c_size_t, ctypes.POINTER(i64)]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [c_int]
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_abi_version.restype = c_int
    lib.fa_abi_version.argtypes = []
    if lib.fa_abi_version() != ABI_VERSION:
        raise FaError(FA_EHIP, f"ABI version {lib.fa_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return fa_status_str(status)
    except FaError:
        return f"status {status}"


# ---- one-to-one mirrors of the C ABI --------------------------------------

def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, d: int,
           dtype: int, mask: int, window: int, scale: float, stream: int | None) -> int:
    """Raw launch on device pointers; returns the fa_status code."""
    return _load().fa_fwd(q, k, v, o, lse, B, H, S, d, dtype, mask, window,
                          ctypes.c_float(scale), stream)


def fa_fwd_gqa(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Hkv: int, S: int,
               d: int, dtype: int, mask: int, window: int, scale: float,
               stream: int | None) -> int:
    """Raw launch with Hkv key/value heads; returns the fa_status code."""
    return _load().fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, S, d, dtype, mask, window,
                              ctypes.c_float(scale), stream)


def fa_bwd(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int,
           delta: int, B: int, H: int, Hkv: int, S: int, d: int, dtype: int, mask: int,
           window: int, scale: float, stream: int | None) -> int:
    """Raw backward launch on device pointers; returns the fa_status code."""
    return _load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, S, d, dtype,
                          mask, window, ctypes.c_float(scale), stream)


def fa_decode_paged(q: int, k_cache: int, v_cache: int, block_table: int, ctx_lens: int,
                    o: int, lse: int, workspace: int | None, workspace_bytes: int, B: int,
                    H: int, Hkv: int, n_q: int, d: int, num_blocks: int, block_size: int,
                    max_blocks: int, max_ctx: int, dtype: int, scale: float,
                    stream: int | None) -> int:
    """Raw paged-cache decode launch on device pointers; returns the status."""
    return _load().fa_decode_paged(q, k_cache, v_cache, block_table, ctx_lens, o, lse,
                                   workspace, workspace_bytes, B, H, Hkv, n_q, d, num_blocks,
                                   block_size, max_blocks, max_ctx, dtype,
                                   ctypes.c_float(scale), stream)


def fa_decode_paged_noalloc(q: int, k_cache: int, v_cache: int, block_table: int,
                            ctx_lens: int, o: int, lse: int, B: int, H: int, Hkv: int, n_q: int,
                            d: int, num_blocks: int, block_size: int, max_blocks: int,
                            max_ctx: int, dtype: int, scale: float, stream: int | None) -> int:
    """Raw paged-cache decode with the library's own split scratch (no
    workspace argument, nothing allocated); returns the status."""
    return _load().fa_decode_paged_noalloc(q, k_cache, v_cache, block_table, ctx_lens, o, lse,
                                           B, H, Hkv, n_q, d, num_blocks, block_size,
                                           max_blocks, max_ctx, dtype, ctypes.c_float(scale),
                                           stream)


def fa_decode_workspace_size(B: int, H: int, Hkv: int, n_q: int, d: int, num_blocks: int,
                             block_size: int, max_blocks: int, max_ctx: int,
                             dtype: int) -> int:
    """Workspace bytes fa_decode_paged needs for these sizes (raises on error)."""
    out = ctypes.c_size_t(0)
    st = _load().fa_decode_workspace_size(B, H, Hkv, n_q, d, num_blocks, block_size,
                                          max_blocks, max_ctx, dtype, ctypes.byref(out))
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return out.value


def fa_query(d: int, dtype: int, mask: int) -> str:
    buf = ctypes.create_string_buffer(128)
    st = _load().fa_query(d, dtype, mask, buf, len(buf))
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return buf.value.decode()


def fa_query_fwd(B: int, H: int, Hkv: int, S: int, d: int, dtype: int, mask: int,
                 window: int = 0) -> tuple[str, int]:
    """(kernel instance, work-groups) that fa_fwd / fa_fwd_gqa would launch
    for these sizes; raises on error."""
    buf = ctypes.create_string_buffer(160)
    grid = ctypes.c_int64(0)
    st = _load().fa_query_fwd(B, H, Hkv, S, d, dtype, mask, window, buf, len(buf),
                              ctypes.byref(grid))
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return buf.value.decode(), grid.value


def fa_status_str(status: int) -> str:
    return _load().fa_status_str(status).decode()


def fa_last_error() -> str:
    return _load().fa_last_error().decode()


def fa_abi_version() -> int:
    return _load().fa_abi_version()


# ---- tensor-level wrapper --------------------------------------------------

def _torch_dtype_code(t) -> int:
    import torch
    codes = {torch.float32: DTYPES["f32"], torch.float16: DTYPES["f16"],
             torch.bfloat16: DTYPES["bf16"]}
    if t.dtype not in codes:
        raise FaError(FA_EINVAL, f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def forward(q, k, v, mask: str = "none", window: int | None = None,
            scale: float | None = None, out=None, lse=None, stream=None):
    """Exact attention forward on [B, H, S, d] device tensors.

    k and v may carry fewer heads than q (grouped-query attention: [B, Hkv, S,
    d] with Hkv dividing H; query head h uses key/value head h // (H // Hkv)).
    Returns (o, lse): o has q's shape and dtype, lse is fp32 [B, H, S] (natural
    log).  ``scale`` defaults to 1/sqrt(d).  Launches on ``stream`` (a torch
    stream) or torch's current stream; asynchronous like any torch op.
    """
    import torch
    if mask not in MASKS:
        raise FaError(FA_EINVAL, f"unknown mask {mask!r}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise FaError(FA_EINVAL, f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise FaError(FA_EINVAL, f"{name} must be a contiguous [B, H, S, d] tensor")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise FaError(FA_EINVAL, "k and v must be [B, Hkv, S, d] with q's B, S and d")
    if not (q.dtype == k.dtype == v.dtype):
        raise FaError(FA_EINVAL, "q, k, v must share a dtype")
    if not (q.device == k.device == v.device):
        raise FaError(FA_EINVAL, "q, k, v must be on one device")
    B, H, S, d = q.shape
    dt = _torch_dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    # A host tensor would pass every check of the C library (which cannot
    # tell host from device pointers) and fault in the kernel's stores.
    for name, t in (("out", out), ("lse", lse)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != q.device:
            raise FaError(FA_EINVAL, f"{name} must be a device tensor on q's device")
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise FaError(FA_EINVAL, "out must match q")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise FaError(FA_EINVAL, "lse must be a contiguous fp32 [B, H, S] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    Hkv = k.shape[1]
    with torch.cuda.device(q.device):
        if Hkv == H:
            st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr(), B, H, S, d, dt, MASKS[mask], int(window or 0),
                        float(scale), stream.cuda_stream)
        else:
            st = fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, H, Hkv, S, d, dt, MASKS[mask],
                            int(window or 0), float(scale), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return out, lse


def backward(q, k, v, o, lse, dout, mask: str = "none", window: int | None = None,
             scale: float | None = None, stream=None):
    """Gradients (dq, dk, dv) of ``forward(q, k, v, mask, window, scale)``.

    ``o`` and ``lse`` are that forward's outputs and ``dout`` the gradient of
    ``o``.  dq has q's shape, dk and dv have k's ([B, Hkv, S, d]; with grouped
    heads they sum over the query heads of each group).  Asynchronous on
    ``stream`` or torch's current stream.
    """
    import torch
    if mask not in MASKS:
        raise FaError(FA_EINVAL, f"unknown mask {mask!r}")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise FaError(FA_EINVAL, f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise FaError(FA_EINVAL, f"{name} must be a contiguous [B, H, S, d] tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise FaError(FA_EINVAL, f"{name} must match q's dtype and device")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise FaError(FA_EINVAL, "k and v must be [B, Hkv, S, d] with q's B, S and d")
    if o.shape != q.shape or dout.shape != q.shape:
        raise FaError(FA_EINVAL, "o and dout must have q's shape")
    B, H, S, d = q.shape
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, S)
            or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device):
        raise FaError(FA_EINVAL, "lse must be a contiguous fp32 [B, H, S] device tensor")
    dt = _torch_dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    delta.data_ptr(), B, H, k.shape[1], S, d, dt, MASKS[mask],
                    int(window or 0), float(scale), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return dq, dk, dv


def decode(q, k_cache, v_cache, block_table, ctx_lens, max_ctx: int, scale: float | None = None,
           stream=None):
    """Attention of q's n_q newest tokens per request over a paged cache.

    q: [B, H, n_q, d]; k_cache, v_cache: [num_blocks, Hkv, block_size, d];
    block_table: int32 [B, max_blocks]; ctx_lens: int32 [B]; all on one
    device.  ``max_ctx`` is a host-side bound on the context lengths.
    Returns (o [B, H, n_q, d], lse fp32 [B, H, n_q]).
    """
    import torch
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("ctx_lens", ctx_lens)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise FaError(FA_EINVAL, f"{name} must be a contiguous device tensor")
        if t.device != q.device:
            raise FaError(FA_EINVAL, f"{name} must be on q's device")
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise FaError(FA_EINVAL, "q must be [B, H, n_q, d] and the caches "
                                 "[num_blocks, Hkv, block_size, d]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise FaError(FA_EINVAL, "q and the caches must share a dtype")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise FaError(FA_EINVAL, "block_table and ctx_lens must be int32")
    B, H, n_q, d = q.shape
    nb, Hkv, bs, d2 = k_cache.shape
    if d2 != d or block_table.dim() != 2 or block_table.shape[0] != B or \
            ctx_lens.shape != (B,):
        raise FaError(FA_EINVAL, "shapes of the caches, block_table or ctx_lens disagree with q")
    dt = _torch_dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mb = block_table.shape[1]
    ws_bytes = fa_decode_workspace_size(B, H, Hkv, n_q, d, nb, bs, mb, int(max_ctx), dt)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = fa_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                             block_table.data_ptr(), ctx_lens.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), ws.data_ptr(), ws.numel(), B, H, Hkv, n_q, d, nb,
                             bs, mb, int(max_ctx), dt, float(scale), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, fa_last_error())
    return o, lse

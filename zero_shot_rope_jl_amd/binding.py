"""ctypes binding of include/jetlong.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(PKG, "libjetlong.so")

JL_OK, JL_EINVAL, JL_EUNSUPPORTED, JL_EHIP, JL_ESPACE = 0, 1, 2, 3, 4
JL_F32, JL_BF16 = 0, 1


class JetLongError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"jetlong error {code}: {message}")
        self.code = code


class JLRotatedKeys(ctypes.Structure):
    """jl_rotated_keys: rows 0..rows-1 of a rotated-key cache hold their keys in
    the remote view under group size G."""
    _fields_ = [("G", ctypes.c_int64), ("rows", ctypes.c_int64)]


def _load():
    # PyTorch-ROCm ships its own HIP runtime (torch/lib/libamdhip64.so).  If
    # libjetlong.so were loaded first, the process would map two HIP/HSA
    # runtimes and the second to initialise would find no device; importing
    # torch first lets the library bind to torch's already-loaded runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build it with `python -m zero_shot_rope_jl_amd.build` "
            "(there is no non-HIP fallback)")
    L = ctypes.CDLL(lib_path)
    i64, sz, vp, cp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p
    L.jl_last_error.restype = cp
    L.jl_last_error.argtypes = []
    L.jl_version.restype = ctypes.c_int
    L.jl_device_info.restype = ctypes.c_int
    L.jl_device_info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.jl_schedule.restype = ctypes.c_int
    L.jl_schedule.argtypes = [i64, i64, i64, ctypes.c_double, ctypes.POINTER(i64), vp, sz,
                              ctypes.POINTER(sz), vp]
    L.jl_table_fill_host.restype = ctypes.c_int
    L.jl_table_fill_host.argtypes = [i64, i64, ctypes.c_double, vp, sz]
    L.jl_bifocal_prefill.restype = ctypes.c_int
    L.jl_bifocal_prefill_workspace.restype = ctypes.c_int
    L.jl_bifocal_prefill_workspace.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.POINTER(sz)]
    L.jl_bifocal_prefill.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                     i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz, vp, sz, vp]
    L.jl_bifocal_prefill_unfused_workspace.restype = ctypes.c_int
    L.jl_bifocal_prefill_unfused_workspace.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                                       ctypes.POINTER(sz)]
    L.jl_bifocal_prefill_unfused.restype = ctypes.c_int
    L.jl_bifocal_prefill_unfused.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                             i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz, vp, sz, vp]
    rk = ctypes.POINTER(JLRotatedKeys)
    L.jl_bifocal_prefill_chunk_paged.restype = ctypes.c_int
    L.jl_bifocal_prefill_chunk_paged.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                                 i64, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                                 ctypes.c_float, vp, sz, vp, sz, rk, vp]
    L.jl_bifocal_prefill_chunk.restype = ctypes.c_int
    L.jl_bifocal_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                           i64, i64, i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz, vp,
                                           sz, rk, vp]
    L.jl_bifocal_prefill_chunk_workspace.restype = ctypes.c_int
    L.jl_bifocal_prefill_chunk_workspace.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64,
                                                     ctypes.POINTER(sz)]
    L.jl_bifocal_decode_workspace.restype = ctypes.c_int
    L.jl_bifocal_decode_workspace.argtypes = [i64, i64, i64, i64, ctypes.POINTER(sz)]
    L.jl_bifocal_decode.restype = ctypes.c_int
    L.jl_bifocal_decode.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                    i64, i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz, vp, sz, vp]
    L.jl_bifocal_decode_noalloc.restype = ctypes.c_int
    L.jl_bifocal_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                            i64, i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz, vp]
    L.jl_bifocal_decode_unfused_workspace.restype = ctypes.c_int
    L.jl_bifocal_decode_unfused_workspace.argtypes = [i64, i64, i64, i64, ctypes.POINTER(sz)]
    L.jl_bifocal_decode_unfused.restype = ctypes.c_int
    L.jl_bifocal_decode_unfused.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                            i64, i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz, vp, sz, vp]
    L.jl_bifocal_decode_rkc.restype = ctypes.c_int
    L.jl_bifocal_decode_rkc.argtypes = [vp, vp, vp, vp, ctypes.POINTER(JLRotatedKeys), vp, vp, ctypes.c_int,
                                        ctypes.c_int, i64, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                        ctypes.c_float, vp, sz, vp, sz, vp]
    L.jl_bifocal_decode_paged.restype = ctypes.c_int
    L.jl_bifocal_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                          i64, i64, i64, i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, sz,
                                          vp, sz, vp]
    L.jl_rope_interleaved_to_half.restype = ctypes.c_int
    L.jl_rope_interleaved_to_half.argtypes = [vp, vp, ctypes.c_int, i64, i64, vp]
    d = ctypes.c_double
    L.jl_fi_table.restype = ctypes.c_int
    L.jl_fi_table.argtypes = [i64, i64, i64, d, d, d, vp, sz, ctypes.POINTER(sz), vp]
    L.jl_fi_table_fill_host.restype = ctypes.c_int
    L.jl_fi_table_fill_host.argtypes = [i64, i64, i64, d, d, d, vp, sz]
    L.jl_bifocal_prefill_fi.restype = ctypes.c_int
    L.jl_bifocal_prefill_fi.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i64,
                                        i64, i64, d, d, d, ctypes.c_float, vp, sz, vp, sz, vp]
    L.jl_bifocal_decode_fi.restype = ctypes.c_int
    L.jl_bifocal_decode_fi.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i64,
                                       i64, i64, i64, d, d, d, ctypes.c_float, vp, sz, vp]
    return L


lib = _load()


def jl_last_error() -> str:
    return lib.jl_last_error().decode()


def jl_version() -> int:
    return lib.jl_version()


def jl_device_info(device: int = 0):
    """(compute units, peak shader clock in kHz) of a HIP device."""
    n, c = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib.jl_device_info(device, ctypes.byref(n), ctypes.byref(c)))
    return n.value, c.value


def _check(rc: int) -> None:
    if rc != JL_OK:
        raise JetLongError(rc, jl_last_error())


# ------------------------------------------------------------ torch helpers
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return JL_BF16
    if t.dtype == torch.float32:
        return JL_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _scratch(nbytes: int, device, stream):
    """Device scratch for one call that allocates it itself.  The caching
    allocator may hand a freed block to the next allocation on the stream it
    was allocated on, so the block is allocated on the stream the call's
    kernels run on: then any reuse is ordered after those kernels.  (Allocated
    on torch's current stream while the kernels run on another, it could be
    reused while they still read or write it.)"""
    torch = _torch()
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _need_device(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


# ------------------------------------------------------------------ the ABI
def jl_schedule(L: int, w_pretrained: int, head_dim: int = 128, rope_base: float = 1e6,
                table=None, stream=None):
    """G = max(1, ceil(L / w_pretrained)) and the table size for (L, head_dim).

    If ``table`` (a uint8 device tensor) is given, the correction table for
    (head_dim, rope_base) covering L positions is filled on the stream.
    Returns (G, table_bytes_needed)."""
    G = ctypes.c_int64(0)
    need = ctypes.c_size_t(0)
    if table is not None:
        _need_device(table)
        rc = lib.jl_schedule(L, w_pretrained, head_dim, rope_base, ctypes.byref(G), _ptr(table),
                             table.numel() * table.element_size(), ctypes.byref(need), _stream(stream))
    else:
        rc = lib.jl_schedule(L, w_pretrained, head_dim, rope_base, ctypes.byref(G), None, 0,
                             ctypes.byref(need), None)
    _check(rc)
    return G.value, need.value


def jl_table_fill_host(L: int, head_dim: int, rope_base: float):
    """Host-built table (numpy uint8 array) with the device table's layout."""
    import numpy as np
    need = ctypes.c_size_t(0)
    _check(lib.jl_schedule(L, 1, head_dim, rope_base, ctypes.byref(ctypes.c_int64(0)), None, 0,
                           ctypes.byref(need), None))
    buf = np.zeros(need.value, dtype=np.uint8)
    _check(lib.jl_table_fill_host(L, head_dim, rope_base, buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes))
    return buf


def alloc_table(L: int, head_dim: int, rope_base: float, device="cuda", stream=None, w_pretrained: int = 1):
    """Allocate a device table with torch and fill it through jl_schedule.

    It serves every call with up to L tokens and pretrained window >=
    ``w_pretrained``; the default 1 covers every window (offsets up to L - 1)."""
    torch = _torch()
    _, need = jl_schedule(L, w_pretrained, head_dim, rope_base)
    t = torch.empty(need, dtype=torch.uint8, device=device)
    jl_schedule(L, w_pretrained, head_dim, rope_base, table=t, stream=stream)
    return t


def jl_bifocal_prefill_workspace(in_dtype: int, B: int, L: int, Hkv: int, D: int, w_pretrained: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.jl_bifocal_prefill_workspace(in_dtype, B, L, Hkv, D, w_pretrained, ctypes.byref(n)))
    return n.value


def alloc_prefill_workspace(k, w_pretrained: int, device="cuda"):
    """Scratch for jl_bifocal_prefill over keys shaped like `k` [B, L, Hkv, D] (None if none is needed)."""
    torch = _torch()
    B, L, Hkv, D = k.shape
    n = jl_bifocal_prefill_workspace(_dtype_code(k), B, L, Hkv, D, w_pretrained)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def jl_bifocal_prefill(q, k, v, out, lse, w0: int, w_pretrained: int, rope_base: float,
                       sm_scale: float, table, workspace=None, stream=None):
    """q [B,L,Hq,D], k/v [B,L,Hkv,D], out [B,L,Hq,D], lse [B,Hq,L] fp32 or None.

    `workspace`: device scratch of jl_bifocal_prefill_workspace bytes (see
    alloc_prefill_workspace); when None and some is needed, one is allocated
    through torch for this call, on the stream the call runs on.
    """
    _need_device(q, k, v, out, lse, table, workspace)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, L, Hkv, D) or tuple(v.shape) != (B, L, Hkv, D):
        raise ValueError("k and v must be [B, L, Hkv, D] matching q")
    if tuple(out.shape) != (B, L, Hq, D):
        raise ValueError("out must be [B, L, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq, L) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq, L]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if workspace is None:
        n = jl_bifocal_prefill_workspace(_dtype_code(k), B, L, Hkv, D, w_pretrained)
        workspace = _scratch(n, q.device, stream) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.jl_bifocal_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                                  _dtype_code(out), B, L, Hq, Hkv, D, w0, w_pretrained, rope_base,
                                  sm_scale, _ptr(table), table.numel() * table.element_size(),
                                  _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def jl_bifocal_prefill_unfused_workspace(in_dtype: int, B: int, L: int, Hq: int, Hkv: int, D: int,
                                         w_pretrained: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.jl_bifocal_prefill_unfused_workspace(in_dtype, B, L, Hq, Hkv, D, w_pretrained, ctypes.byref(n)))
    return n.value


def alloc_prefill_unfused_workspace(q, k, w_pretrained: int, device="cuda"):
    """Scratch for jl_bifocal_prefill_unfused over q [B, L, Hq, D] and k [B, L, Hkv, D]."""
    torch = _torch()
    B, L, Hq, D = q.shape
    n = jl_bifocal_prefill_unfused_workspace(_dtype_code(q), B, L, Hq, k.shape[2], D, w_pretrained)
    return torch.empty(n, dtype=torch.uint8, device=device)


def jl_bifocal_prefill_unfused(q, k, v, out, lse, w0: int, w_pretrained: int, rope_base: float,
                               sm_scale: float, table, workspace=None, stream=None):
    """The three-pass form of jl_bifocal_prefill (same arguments); `workspace`
    as from alloc_prefill_unfused_workspace, allocated through torch if None."""
    _need_device(q, k, v, out, lse, table, workspace)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, L, Hkv, D) or tuple(v.shape) != (B, L, Hkv, D):
        raise ValueError("k and v must be [B, L, Hkv, D] matching q")
    if tuple(out.shape) != (B, L, Hq, D):
        raise ValueError("out must be [B, L, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq, L) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq, L]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if workspace is None:
        workspace = _scratch(jl_bifocal_prefill_unfused_workspace(_dtype_code(q), B, L, Hq, Hkv, D, w_pretrained),
                             q.device, stream)
    _check(lib.jl_bifocal_prefill_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                                          _dtype_code(out), B, L, Hq, Hkv, D, w0, w_pretrained, rope_base,
                                          sm_scale, _ptr(table), table.numel() * table.element_size(),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
    return out, lse


def jl_bifocal_prefill_chunk_workspace(in_dtype: int, B: int, Lq: int, Lcap: int, Hq: int, Hkv: int, D: int,
                                       w_pretrained: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.jl_bifocal_prefill_chunk_workspace(in_dtype, B, Lq, Lcap, Hq, Hkv, D, w_pretrained, ctypes.byref(n)))
    return n.value


class ChunkState:
    """A chunk workspace with its rotated-key state (jl_rotated_keys): pass
    the same one to the chunks of one sequence so that each chunk rotates
    only its new keys.  Call reset() after rewriting cached keys."""

    def __init__(self, nbytes: int, device="cuda"):
        torch = _torch()
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None
        self.state = JLRotatedKeys(0, 0)

    def reset(self):
        self.state.G = 0
        self.state.rows = 0


def alloc_chunk_state(q, k_cache, w_pretrained: int, Lq_max: int | None = None, device="cuda"):
    """ChunkState for chunks of up to Lq_max tokens (default: q's) over k_cache [B, Lcap, Hkv, D]."""
    B, Lq, Hq, D = q.shape
    Lcap, Hkv = k_cache.shape[1], k_cache.shape[2]
    n = jl_bifocal_prefill_chunk_workspace(_dtype_code(q), B, Lq_max or Lq, Lcap, Hq, Hkv, D, w_pretrained)
    return ChunkState(n, device)


def _chunk_ws(workspace, nbytes, device, stream):
    """(device buffer, state pointer) of a chunk call's workspace argument: a
    ChunkState, a plain tensor (no state: every key row rotated), or None (a
    buffer for this call on its stream)."""
    if isinstance(workspace, ChunkState):
        return workspace.buf, ctypes.byref(workspace.state)
    if workspace is None and nbytes:
        workspace = _scratch(nbytes, device, stream)
    return workspace, None


def jl_bifocal_prefill_chunk(q, k_cache, v_cache, out, lse, L: int, w0: int, w_pretrained: int,
                             rope_base: float, sm_scale: float, table, workspace=None, stream=None):
    """q [B,Lq,Hq,D] at positions L-Lq..L-1, caches [B,Lmax,Hkv,D] with rows < L valid,
    out [B,Lq,Hq,D], lse [B,Hq,Lq] fp32 or None.  `workspace`: a ChunkState (see
    alloc_chunk_state; keeps the rotated keys across the chunks of a sequence), a
    device tensor of jl_bifocal_prefill_chunk_workspace bytes, or None (allocated
    through torch for this call)."""
    B, Lq, Hq, D = q.shape
    Bk, Lmax, Hkv, Dk = k_cache.shape
    buf0 = workspace.buf if isinstance(workspace, ChunkState) else workspace
    _need_device(q, k_cache, v_cache, out, lse, table, buf0)
    if Bk != B or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [B, Lmax, Hkv, D] matching q")
    if tuple(out.shape) != (B, Lq, Hq, D):
        raise ValueError("out must be [B, Lq, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq, Lq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq, Lq]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    n = jl_bifocal_prefill_chunk_workspace(_dtype_code(q), B, Lq, Lmax, Hq, Hkv, D, w_pretrained)
    buf, st = _chunk_ws(workspace, n, q.device, stream)
    ws_bytes = 0 if buf is None else buf.numel() * buf.element_size()
    _check(lib.jl_bifocal_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                        _dtype_code(q), _dtype_code(out), B, Lq, L, Lmax, Hq, Hkv, D, w0,
                                        w_pretrained, rope_base, sm_scale, _ptr(table),
                                        table.numel() * table.element_size(), _ptr(buf), ws_bytes, st,
                                        _stream(stream)))
    return out, lse


def jl_bifocal_prefill_chunk_paged(q, k_pages, v_pages, block_table, out, lse, L: int, w0: int, w_pretrained: int,
                                   rope_base: float, sm_scale: float, table, workspace=None, stream=None):
    """q [B,Lq,Hq,D] bf16 at positions L-Lq..L-1; pages [n_pages, page_size, Hkv, D] bf16;
    block_table [B, max_pages] int32; out [B,Lq,Hq,D]; lse [B,Hq,Lq] fp32 or None.
    `workspace` as for jl_bifocal_prefill_chunk, sized for max_pages * page_size rows."""
    torch = _torch()
    B, Lq, Hq, D = q.shape
    n_pages, page_size, Hkv, Dk = k_pages.shape
    buf0 = workspace.buf if isinstance(workspace, ChunkState) else workspace
    _need_device(q, k_pages, v_pages, block_table, out, lse, table, buf0)
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("the pages must be [n_pages, page_size, Hkv, D] matching q")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if tuple(out.shape) != (B, Lq, Hq, D):
        raise ValueError("out must be [B, Lq, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq, Lq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq, Lq]")
    max_pages = block_table.shape[1]
    n = jl_bifocal_prefill_chunk_workspace(_dtype_code(q), B, Lq, max_pages * page_size, Hq, Hkv, D, w_pretrained)
    buf, st = _chunk_ws(workspace, n, q.device, stream)
    ws_bytes = 0 if buf is None else buf.numel() * buf.element_size()
    _check(lib.jl_bifocal_prefill_chunk_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(out),
                                              _ptr(lse), _dtype_code(q), _dtype_code(out), B, Lq, L, n_pages,
                                              page_size, max_pages, Hq, Hkv, D, w0, w_pretrained, rope_base,
                                              sm_scale, _ptr(table), table.numel() * table.element_size(),
                                              _ptr(buf), ws_bytes, st, _stream(stream)))
    return out, lse


def jl_bifocal_decode_workspace(B: int, Hq: int, D: int, L: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.jl_bifocal_decode_workspace(B, Hq, D, L, ctypes.byref(n)))
    return n.value


def alloc_decode_workspace(B: int, Hq: int, D: int, Lmax: int, device="cuda"):
    """Decode workspace (split partials) for steps of up to Lmax keys."""
    torch = _torch()
    n = jl_bifocal_decode_workspace(B, Hq, D, Lmax)
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def jl_bifocal_decode_unfused_workspace(B: int, Hq: int, D: int, L: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.jl_bifocal_decode_unfused_workspace(B, Hq, D, L, ctypes.byref(n)))
    return n.value


def alloc_decode_unfused_workspace(B: int, Hq: int, D: int, Lmax: int, device="cuda"):
    """Workspace of jl_bifocal_decode_unfused for steps of up to Lmax keys."""
    torch = _torch()
    n = jl_bifocal_decode_unfused_workspace(B, Hq, D, Lmax)
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def jl_bifocal_decode(q, k_cache, v_cache, out, lse, L: int, w0: int, w_pretrained: int,
                      rope_base: float, sm_scale: float, table, workspace, stream=None):
    """q [B,1,Hq,D] bf16, caches [B,Lmax,Hkv,D] bf16, out [B,1,Hq,D], lse [B,Hq] or None."""
    _need_device(q, k_cache, v_cache, out, lse, table, workspace)
    B, one, Hq, D = q.shape
    _, Lmax, Hkv, Dk = k_cache.shape
    if one != 1 or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("q must be [B,1,Hq,D] and the caches [B,Lmax,Hkv,D]")
    if tuple(out.shape) != (B, 1, Hq, D):
        raise ValueError("out must be [B, 1, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq]")
    _check(lib.jl_bifocal_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                 _dtype_code(q), _dtype_code(out), B, L, Lmax, Hq, Hkv, D, w0,
                                 w_pretrained, rope_base, sm_scale, _ptr(table),
                                 table.numel() * table.element_size(), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def jl_bifocal_decode_noalloc(q, k_cache, v_cache, out, lse, L: int, w0: int, w_pretrained: int,
                              rope_base: float, sm_scale: float, table, stream=None):
    """jl_bifocal_decode with the library's fixed scratch instead of a
    workspace (no allocation anywhere in the call)."""
    _need_device(q, k_cache, v_cache, out, lse, table)
    B, one, Hq, D = q.shape
    _, Lmax, Hkv, Dk = k_cache.shape
    if one != 1 or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("q must be [B,1,Hq,D] and the caches [B,Lmax,Hkv,D]")
    if tuple(out.shape) != (B, 1, Hq, D):
        raise ValueError("out must be [B, 1, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq]")
    _check(lib.jl_bifocal_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                         _dtype_code(q), _dtype_code(out), B, L, Lmax, Hq, Hkv, D, w0,
                                         w_pretrained, rope_base, sm_scale, _ptr(table),
                                         table.numel() * table.element_size(), _stream(stream)))
    return out, lse


def jl_bifocal_decode_unfused(q, k_cache, v_cache, out, lse, L: int, w0: int, w_pretrained: int,
                              rope_base: float, sm_scale: float, table, workspace, stream=None):
    """jl_bifocal_decode computed as three passes and their §3.3 Eq. 6 merge;
    `workspace` from alloc_decode_unfused_workspace."""
    _need_device(q, k_cache, v_cache, out, lse, table, workspace)
    B, one, Hq, D = q.shape
    _, Lmax, Hkv, Dk = k_cache.shape
    if one != 1 or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("q must be [B,1,Hq,D] and the caches [B,Lmax,Hkv,D]")
    if tuple(out.shape) != (B, 1, Hq, D):
        raise ValueError("out must be [B, 1, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq]")
    _check(lib.jl_bifocal_decode_unfused(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                         _dtype_code(q), _dtype_code(out), B, L, Lmax, Hq, Hkv, D, w0,
                                         w_pretrained, rope_base, sm_scale, _ptr(table),
                                         table.numel() * table.element_size(), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


class RotatedKeyCache:
    """A rotated-key cache for jl_bifocal_decode_rkc: device keys laid out like
    the key cache they cover, and the host state the library keeps current.
    Call reset() after rewriting rows of the key cache that it covers."""

    def __init__(self, k_cache):
        self.keys = _torch().empty_like(k_cache)
        self.state = JLRotatedKeys(0, 0)

    def reset(self):
        self.state.G = 0
        self.state.rows = 0


def jl_bifocal_decode_rkc(q, k_cache, v_cache, rkc, out, lse, L: int, w0: int, w_pretrained: int,
                          rope_base: float, sm_scale: float, table, workspace, stream=None):
    """jl_bifocal_decode with the remote keys read from `rkc` (a RotatedKeyCache
    of k_cache), which the call brings up to date first."""
    _need_device(q, k_cache, v_cache, rkc.keys, out, lse, table, workspace)
    B, one, Hq, D = q.shape
    _, Lmax, Hkv, Dk = k_cache.shape
    if one != 1 or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("q must be [B,1,Hq,D] and the caches [B,Lmax,Hkv,D]")
    if tuple(rkc.keys.shape) != tuple(k_cache.shape) or rkc.keys.dtype != k_cache.dtype:
        raise ValueError("the rotated-key cache must match k_cache")
    if tuple(out.shape) != (B, 1, Hq, D):
        raise ValueError("out must be [B, 1, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq]")
    _check(lib.jl_bifocal_decode_rkc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(rkc.keys),
                                     ctypes.byref(rkc.state), _ptr(out), _ptr(lse), _dtype_code(q),
                                     _dtype_code(out), B, L, Lmax, Hq, Hkv, D, w0, w_pretrained, rope_base,
                                     sm_scale, _ptr(table), table.numel() * table.element_size(), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def jl_bifocal_decode_paged(q, k_pages, v_pages, block_table, out, lse, L: int, w0: int, w_pretrained: int,
                            rope_base: float, sm_scale: float, table, workspace, stream=None):
    """q [B,1,Hq,D] bf16; pages [n_pages, page_size, Hkv, D] bf16; block_table [B, max_pages] int32;
    out [B,1,Hq,D]; lse [B,Hq] or None."""
    torch = _torch()
    _need_device(q, k_pages, v_pages, block_table, out, lse, table, workspace)
    B, one, Hq, D = q.shape
    n_pages, page_size, Hkv, Dk = k_pages.shape
    if one != 1 or Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("q must be [B,1,Hq,D] and the pages [n_pages, page_size, Hkv, D]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if tuple(out.shape) != (B, 1, Hq, D):
        raise ValueError("out must be [B, 1, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq]")
    _check(lib.jl_bifocal_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(out),
                                       _ptr(lse), _dtype_code(q), _dtype_code(out), B, L, n_pages, page_size,
                                       block_table.shape[1], Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale,
                                       _ptr(table), table.numel() * table.element_size(), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


# ---- frequency-interpolation remote view (the §4.7 ablation) -------------
def jl_fi_table(L: int, w_pretrained: int, head_dim: int, rope_base: float, fi_alpha: float, fi_beta: float,
                table=None, stream=None) -> int:
    """Size of the interpolation table for this call; fills ``table`` (a
    uint8 device tensor) on the stream when given."""
    need = ctypes.c_size_t(0)
    if table is not None:
        _need_device(table)
        rc = lib.jl_fi_table(L, w_pretrained, head_dim, rope_base, fi_alpha, fi_beta, _ptr(table),
                             table.numel() * table.element_size(), ctypes.byref(need), _stream(stream))
    else:
        rc = lib.jl_fi_table(L, w_pretrained, head_dim, rope_base, fi_alpha, fi_beta, None, 0,
                             ctypes.byref(need), None)
    _check(rc)
    return need.value


def jl_fi_table_fill_host(L: int, w_pretrained: int, head_dim: int, rope_base: float, fi_alpha: float,
                          fi_beta: float):
    """Host-built interpolation table (numpy uint8 array), the device layout."""
    import numpy as np
    buf = np.zeros(jl_fi_table(L, w_pretrained, head_dim, rope_base, fi_alpha, fi_beta), dtype=np.uint8)
    _check(lib.jl_fi_table_fill_host(L, w_pretrained, head_dim, rope_base, fi_alpha, fi_beta,
                                     buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes))
    return buf


def alloc_fi_table(L: int, w_pretrained: int, head_dim: int, rope_base: float, fi_alpha: float, fi_beta: float,
                   device="cuda", stream=None):
    """Allocate a device interpolation table with torch and fill it."""
    torch = _torch()
    t = torch.empty(jl_fi_table(L, w_pretrained, head_dim, rope_base, fi_alpha, fi_beta), dtype=torch.uint8,
                    device=device)
    jl_fi_table(L, w_pretrained, head_dim, rope_base, fi_alpha, fi_beta, table=t, stream=stream)
    return t


def jl_bifocal_prefill_fi(q, k, v, out, lse, w0: int, w_pretrained: int, rope_base: float, fi_alpha: float,
                          fi_beta: float, sm_scale: float, table, workspace=None, stream=None):
    """jl_bifocal_prefill with the remote pairs in the frequency-interpolation
    view; ``table`` from alloc_fi_table for this (L, w_pretrained, ramp)."""
    _need_device(q, k, v, out, lse, table, workspace)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, L, Hkv, D) or tuple(v.shape) != (B, L, Hkv, D):
        raise ValueError("k and v must be [B, L, Hkv, D] matching q")
    if tuple(out.shape) != (B, L, Hq, D):
        raise ValueError("out must be [B, L, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq, L) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq, L]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if workspace is None:
        n = jl_bifocal_prefill_workspace(_dtype_code(k), B, L, Hkv, D, w_pretrained)
        workspace = _scratch(n, q.device, stream) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.jl_bifocal_prefill_fi(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                                     _dtype_code(out), B, L, Hq, Hkv, D, w0, w_pretrained, rope_base, fi_alpha,
                                     fi_beta, sm_scale, _ptr(table), table.numel() * table.element_size(),
                                     _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def jl_bifocal_decode_fi(q, k_cache, v_cache, out, lse, L: int, w0: int, w_pretrained: int, rope_base: float,
                         fi_alpha: float, fi_beta: float, sm_scale: float, workspace, stream=None):
    """jl_bifocal_decode with the remote keys in the frequency-interpolation
    view for this L (no table)."""
    _need_device(q, k_cache, v_cache, out, lse, workspace)
    B, one, Hq, D = q.shape
    _, Lmax, Hkv, Dk = k_cache.shape
    if one != 1 or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B:
        raise ValueError("q must be [B,1,Hq,D] and the caches [B,Lmax,Hkv,D]")
    if tuple(out.shape) != (B, 1, Hq, D):
        raise ValueError("out must be [B, 1, Hq, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or _dtype_code(lse) != JL_F32):
        raise ValueError("lse must be float32 [B, Hq]")
    _check(lib.jl_bifocal_decode_fi(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _dtype_code(q),
                                    _dtype_code(out), B, L, Lmax, Hq, Hkv, D, w0, w_pretrained, rope_base, fi_alpha,
                                    fi_beta, sm_scale, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def jl_rope_interleaved_to_half(x, out=None, stream=None):
    """Channels of q or k [..., D] from interleaved RoPE pairs (2i, 2i+1) to
    the rotate-half pairs (i, i + D/2); apply to q and k, not v."""
    if out is None:
        out = _torch().empty_like(x)
    _need_device(x, out)
    if tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype:
        raise ValueError("out must match x")
    if not x.is_contiguous() or not out.is_contiguous():
        raise ValueError("x and out must be contiguous")
    D = x.shape[-1]
    _check(lib.jl_rope_interleaved_to_half(_ptr(x), _ptr(out), _dtype_code(x), x.numel() // D, D,
                                           _stream(stream)))
    return out

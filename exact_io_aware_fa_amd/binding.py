"""Thin ctypes binding over ``libfa.so`` (declared in ``include/fa.h``).

Argument marshalling only: every step of the attention forward runs in the
library's HIP kernels.  Torch supplies device memory and the current stream.
If the library is missing, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libfa.so"

FA_F32, FA_BF16 = 0, 1
FA_OK = 0
ABI_VERSION = 5

_lib = None


class FaError(RuntimeError):
    """A non-OK status from the library (message: status name and detail)."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(detail)


def library_path() -> str:
    """The in-tree build; FA_LIBRARY names another build of the same library."""
    return os.environ.get("FA_LIBRARY") or os.path.join(_PKG, _LIBNAME)


def load_library():
    """Load libfa.so once and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(library_path())
    return _lib


def open_library(path: str):
    """Load one build of the library (its own copy of every kernel) and
    declare its C signatures; the calls below use the one load_library()
    returns.  Raises if the file is missing or its ABI version differs."""
    if not os.path.exists(path):
        raise RuntimeError(
            "%s is not built; run __graft_entry__.build() or "
            "python -m exact_io_aware_fa_amd.build" % path)
    lib = ctypes.CDLL(path)
    p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [i32, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, p]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_varlen.argtypes = [i32, p, p, p, p, p, i32, i32, i32, i32, p, p, i32, i32, i32, i32, i32, f32, p]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_decode.argtypes = [i32, p, p, p, p, i32, p, p, i32, i32, i32, i32, f32, p, sz, p]
    lib.fa_decode.restype = i32
    lib.fa_decode_noalloc.argtypes = [i32, p, p, p, p, i32, p, p, i32, i32, i32, i32, f32, p]
    lib.fa_decode_noalloc.restype = i32
    lib.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_paged.argtypes = [i32, p, p, p, p, p, p, p, i32, i32, i32, i32, p, p, i32, i32, i32, i32, f32,
                                    p, sz, p]
    lib.fa_decode_paged.restype = i32
    lib.fa_decode_paged_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_decode_paged_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [i32, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, p, sz, p]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i32
    if lib.fa_abi_version() != ABI_VERSION:
        raise RuntimeError("%s: ABI version %d, binding expects %d"
                           % (path, lib.fa_abi_version(), ABI_VERSION))
    return lib


def abi_version() -> int:
    return load_library().fa_abi_version()


def _raise(lib, st: int):
    name = lib.fa_status_str(st).decode()
    detail = lib.fa_last_error().decode()
    raise FaError(st, "%s: %s" % (name, detail) if detail else name)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError("fa supports bfloat16 and float32 tensors, got %s" % t.dtype)


def _dev_ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fa expects device tensors")
    if not t.is_contiguous():
        raise ValueError("fa expects contiguous tensors")
    return t.data_ptr()


def _check_out(t: torch.Tensor, name: str, shape, dtype, like: torch.Tensor):
    """A caller-given output must be exactly what the kernels write: the C ABI
    receives only its pointer, so a smaller or differently typed buffer would
    be written past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != like.device:
        raise ValueError("%s must be on %s, got %s" % (name, like.device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_same_dtype(ref: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t is not None and t.dtype != ref.dtype:
            raise TypeError("%s must share q's dtype %s, got %s" % (name, ref.dtype, t.dtype))


def _check_workspace(ws: torch.Tensor, like: torch.Tensor):
    if ws.device != like.device:
        raise ValueError("workspace must be on %s, got %s" % (like.device, ws.device))
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _stream_handle(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool, scale: float,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """Prefill forward.  q [B,N,Hq,d], k/v [B,Nk,Hkv,d] -> (o [B,N,Hq,d], lse [B,Hq,N] fp32)."""
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D BSHD tensors")
    B, N, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    _check_same_dtype(q, k=k, v=v)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, q.dtype, q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (B, Hq, N), torch.float32, q)
    st = lib.fa_fwd(_dtype_code(q), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(out),
                    _dev_ptr(lse), B, Hq, Hkv, N, Nk, d, 1 if causal else 0, float(scale),
                    _stream_handle(stream))
    if st != FA_OK:
        _raise(lib, st)
    return out, lse


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, causal: bool, scale: float,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """Varlen / chunked prefill.  q [total_q,Hq,d], k/v [total_k,Hkv,d] (bf16, packed),
    cu_seqlens_q/k int32 [B+1] on the device -> (o [total_q,Hq,d], lse [Hq,total_q] fp32)."""
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [total_q,Hq,d] and k, v [total_k,Hkv,d]")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    if dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    _check_same_dtype(q, k=k, v=v)
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu.dtype != torch.int32 or cu.dim() != 1:
            raise ValueError("%s must be a 1-D int32 tensor" % name)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B+1 entries")
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, q.dtype, q)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (Hq, total_q), torch.float32, q)
    st = lib.fa_fwd_varlen(_dtype_code(q), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(cu_seqlens_q),
                           _dev_ptr(cu_seqlens_k), int(max_seqlen_q), int(max_seqlen_k), total_q, total_k,
                           _dev_ptr(out), _dev_ptr(lse), B, Hq, Hkv, d, 1 if causal else 0, float(scale),
                           _stream_handle(stream))
    if st != FA_OK:
        _raise(lib, st)
    return out, lse


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, max_seqlen_k: int) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, Hq, Hkv, d, max_seqlen_k))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           cu_seqlens_k: torch.Tensor, max_seqlen_k: int, scale: float,
           out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, stream=None):
    """Varlen decode.  q [B,Hq,d], caches [total,Hkv,d], cu_seqlens_k int32 [B+1] (device)
    -> (o [B,Hq,d], lse [B,Hq] fp32).  ``workspace`` is a uint8 device tensor of at
    least ``decode_workspace_bytes`` bytes; one is allocated when omitted."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 3 or v_cache.dim() != 3:
        raise ValueError("q must be [B,Hq,d] and caches [total,Hkv,d]")
    B, Hq, d = q.shape
    total, Hkv, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and caches")
    if cu_seqlens_k.dtype != torch.int32 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_k must be int32 with B+1 entries")
    _check_same_dtype(q, k_cache=k_cache, v_cache=v_cache)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, q.dtype, q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (B, Hq), torch.float32, q)
    # no sequence can be longer than the cache holds rows
    max_seqlen_k = min(int(max_seqlen_k), total)
    need = int(lib.fa_decode_workspace_bytes(B, Hq, Hkv, d, max_seqlen_k))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    st = lib.fa_decode(_dtype_code(q), _dev_ptr(q), _dev_ptr(k_cache), _dev_ptr(v_cache),
                       _dev_ptr(cu_seqlens_k), int(max_seqlen_k), _dev_ptr(out), _dev_ptr(lse),
                       B, Hq, Hkv, d, float(scale), _dev_ptr(workspace),
                       workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != FA_OK:
        _raise(lib, st)
    return out, lse



DECODE_SCRATCH_BYTES = 16 << 20     # FA_DECODE_SCRATCH_BYTES in include/fa.h


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   cu_seqlens_k: torch.Tensor, max_seqlen_k: int, scale: float,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """``decode`` without a workspace argument: the partial results go to the
    library's static device array (fa_decode_noalloc).  With ``out`` and ``lse``
    given the call allocates nothing.  Calls that overlap on one GPU race on
    that array; order them on one stream."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 3 or v_cache.dim() != 3:
        raise ValueError("q must be [B,Hq,d] and caches [total,Hkv,d]")
    B, Hq, d = q.shape
    total, Hkv, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and caches")
    if cu_seqlens_k.dtype != torch.int32 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_k must be int32 with B+1 entries")
    _check_same_dtype(q, k_cache=k_cache, v_cache=v_cache)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, q.dtype, q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (B, Hq), torch.float32, q)
    max_seqlen_k = min(int(max_seqlen_k), total)
    st = lib.fa_decode_noalloc(_dtype_code(q), _dev_ptr(q), _dev_ptr(k_cache), _dev_ptr(v_cache),
                               _dev_ptr(cu_seqlens_k), int(max_seqlen_k), _dev_ptr(out), _dev_ptr(lse),
                               B, Hq, Hkv, d, float(scale), _stream_handle(stream))
    if st != FA_OK:
        _raise(lib, st)
    return out, lse

def decode_paged_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, max_seqlen_k: int) -> int:
    return int(load_library().fa_decode_paged_workspace_bytes(B, Hq, Hkv, d, max_seqlen_k))


def decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 seqlens_k: torch.Tensor, max_seqlen_k: int, scale: float, k_new: torch.Tensor | None = None,
                 v_new: torch.Tensor | None = None, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None):
    """Paged decode, appending the new token's rows first when k_new/v_new are given.
    q [B,Hq,d]; caches [num_blocks,block_size,Hkv,d] (updated in place); block_table int32
    [B,max_blocks]; seqlens_k int32 [B] (rows before the append); k_new/v_new [B,Hkv,d]
    -> (o [B,Hq,d], lse [B,Hq] fp32)."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B,Hq,d] and caches [num_blocks,block_size,Hkv,d]")
    B, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and caches")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None and (tuple(k_new.shape) != (B, Hkv, d) or tuple(v_new.shape) != (B, Hkv, d)):
        raise ValueError("k_new and v_new must be [B,Hkv,d]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if seqlens_k.dtype != torch.int32 or seqlens_k.numel() != B:
        raise ValueError("seqlens_k must be int32 with B entries")
    _check_same_dtype(q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, q.dtype, q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (B, Hq), torch.float32, q)
    need = int(lib.fa_decode_paged_workspace_bytes(B, Hq, Hkv, d, int(max_seqlen_k)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    st = lib.fa_decode_paged(_dtype_code(q), _dev_ptr(q), _dev_ptr(k_new), _dev_ptr(v_new), _dev_ptr(k_cache),
                             _dev_ptr(v_cache), _dev_ptr(block_table), _dev_ptr(seqlens_k), num_blocks, block_size,
                             block_table.shape[1], int(max_seqlen_k), _dev_ptr(out), _dev_ptr(lse), B, Hq, Hkv, d,
                             float(scale), _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream_handle(stream))
    if st != FA_OK:
        _raise(lib, st)
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
        causal: bool, scale: float, dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
        dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Backward of ``fwd``: q, o, dout [B,N,Hq,d], k, v [B,Nk,Hkv,d] (bf16), lse [B,Hq,N] fp32
    -> (dq, dk, dv) in the layouts of q, k, v."""
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D BSHD tensors")
    B, N, Hq, d = q.shape
    Bk, Nk, Hkv, dk_ = k.shape
    if Bk != B or dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(lse.shape) != (B, Hq, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, Hq, N]")
    _check_same_dtype(q, k=k, v=v, o=o, dout=dout)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_out(dq, "dq", q.shape, q.dtype, q)
    _check_out(dk, "dk", k.shape, q.dtype, q)
    _check_out(dv, "dv", v.shape, q.dtype, q)
    need = int(lib.fa_bwd_workspace_bytes(B, Hq, N))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    st = lib.fa_bwd(_dtype_code(q), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(lse),
                    _dev_ptr(dout), _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv), B, Hq, Hkv, N, Nk, d,
                    1 if causal else 0, float(scale), _dev_ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != FA_OK:
        _raise(lib, st)
    return dq, dk, dv

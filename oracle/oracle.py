"""Python side of the fp64 CPU oracle (ctypes over ``oracle/liboracle.so``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The GPU path
(``exact_io_aware_fa_amd``) never imports it, and this module imports nothing
from that package.

The forward arithmetic lives in ``oracle.c`` (plain C, fp64, the textbook
definition of attention: S = scale*Q K^T, mask, softmax, P V, LSE = m + ln l);
this file passes the stored bit patterns of the inputs (f64, f32 or bf16) to C,
which widens them exactly.  The compositions here (varlen prefill, decode after
an append) only slice and concatenate inputs around those calls.  The backward
(``attention_bwd``) is the chain rule of the same definition in float64 numpy,
with library matrix products.

Sources: ai6s.net page, sections "standard attention's fatal flaw is data
movement, not compute" and "FlashAttention changes the dataflow, not the
algorithm" (the result equals standard attention); same page, section "what
ops-transformer adds" (causal mask, variable-length KV cache).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2
_ERRORS = {1: "invalid argument", 2: "softmax row sum differs from 1 by more than 1e-12",
           3: "out of memory"}

_default = None

# Worker threads when the caller does not say: the CPUs this process may use,
# capped at 16 (the host share of one GPU on a shared node).
DEFAULT_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source into a shared library with gcc (fp64, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-pthread", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_attn_rows.argtypes = [i32, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                     f64, i64, p, p, p, p, p, i32]
    lib.oracle_attn_rows.restype = i32
    lib.oracle_decode_rows.argtypes = [i32, p, p, p, p, i32, i32, i32, i32, f64,
                                       i64, p, p, p, p, i32]
    lib.oracle_decode_rows.restype = i32
    lib.oracle_version.restype = i32
    return lib


def _load():
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _default = _bind(_LIB)
    return _default


def load_library(path: str):
    """Bind another build of an oracle source (used to check that the pins catch
    deliberately planted mistakes); pass the handle as ``lib=``."""
    return _bind(path)


def _stored(t) -> tuple[np.ndarray, int]:
    """Contiguous host array holding the stored bits of ``t`` and its dtype code."""
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(t)
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float64:
        return t.numpy(), F64
    if t.dtype == torch.float32:
        return t.numpy(), F32
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), BF16
    raise TypeError("oracle inputs must be float64, float32 or bfloat16, got %s" % t.dtype)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _threads(n: int) -> int:
    return int(n) if n and n > 0 else DEFAULT_THREADS


def _check(rc: int):
    if rc != 0:
        raise RuntimeError("oracle failed: " + _ERRORS.get(rc, "code %d" % rc))


def attention_rows(q, k, v, causal: bool, scale: float, rows, nthreads: int = 0, lib=None):
    """Prefill attention for selected query rows.

    q [B,N,Hq,d], k/v [B,Nk,Hkv,d] (same dtype); ``rows`` is an int array of
    shape [R,3] holding (b, h, i).  Returns (o [R,d] float64, lse [R] float64).
    ``scale`` is used as given (pass the fp32 value the GPU receives).
    """
    qa, dt = _stored(q)
    ka, dk = _stored(k)
    va, dv = _stored(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share a dtype")
    B, N, Hq, d = qa.shape
    Bk, Nk, Hkv, dk_ = ka.shape
    if Bk != B or dk_ != d or va.shape != ka.shape:
        raise ValueError("shape mismatch between q, k and v")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    rb = np.ascontiguousarray(rows[:, 0].astype(np.int32))
    rh = np.ascontiguousarray(rows[:, 1].astype(np.int32))
    ri = np.ascontiguousarray(rows[:, 2].astype(np.int32))
    R = rows.shape[0]
    o = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros((R,), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), B, Hq, Hkv, N, Nk, d,
                                  1 if causal else 0, float(scale), R, _ptr(rb), _ptr(rh),
                                  _ptr(ri), _ptr(o), _ptr(lse), _threads(nthreads))
    _check(rc)
    return o, lse


def attention(q, k, v, causal: bool, scale: float, nthreads: int = 0, lib=None):
    """Full prefill attention.  Returns (o [B,N,Hq,d] float64, lse [B,Hq,N] float64)."""
    B, N, Hq, d = q.shape
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(N), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)   # ordered (b, h, i)
    o, lse = attention_rows(q, k, v, causal, scale, rows, nthreads, lib)
    o = o.reshape(B, Hq, N, d).transpose(0, 2, 1, 3).copy()
    lse = lse.reshape(B, Hq, N)
    return o, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool, scale: float, nthreads: int = 0,
                     lib=None):
    """Variable-length prefill: the definition applied to each sequence on its own.

    q [total_q,Hq,d], k/v [total_k,Hkv,d] packed; sequence b owns the q rows
    cu_seqlens_q[b]..cu_seqlens_q[b+1]-1 and the k/v rows cu_seqlens_k[b]..
    cu_seqlens_k[b+1]-1 and is attended as a batch of one (bottom-right causal
    alignment within the sequence).  Source: ai6s.net page, section "what
    ops-transformer adds", second item (causal mask) and third item (attend to
    the real lengths only).  Returns (o [total_q,Hq,d] float64, lse [Hq,total_q]
    float64); rows of no sequence stay 0.
    """
    cq = [int(x) for x in torch.as_tensor(cu_seqlens_q).cpu().tolist()]
    ck = [int(x) for x in torch.as_tensor(cu_seqlens_k).cpu().tolist()]
    if len(cq) != len(ck) or not cq:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B+1 entries")
    total_q, Hq, d = q.shape
    total_k = k.shape[0]
    if cq[-1] > total_q or ck[-1] > total_k:
        raise ValueError("cu_seqlens end past the packed tensors")
    o = np.zeros((total_q, Hq, d), dtype=np.float64)
    lse = np.zeros((Hq, total_q), dtype=np.float64)
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe == qs:
            continue
        ob, lb = attention(q[qs:qe].unsqueeze(0), k[ks:ke].unsqueeze(0), v[ks:ke].unsqueeze(0), causal, scale,
                           nthreads, lib)
        o[qs:qe] = ob[0]
        lse[:, qs:qe] = lb[0]
    return o, lse


def decode_rows(q, k_cache, v_cache, cu_seqlens, scale: float, rows, nthreads: int = 0,
                lib=None):
    """Decode attention for selected (b, h) pairs.

    q [B,Hq,d]; k_cache/v_cache [total,Hkv,d]; cu_seqlens int [B+1] (host);
    ``rows`` int array [R,2] of (b, h).  Returns (o [R,d], lse [R]) in float64.
    """
    qa, dt = _stored(q)
    ka, dk = _stored(k_cache)
    va, dv = _stored(v_cache)
    if not (dt == dk == dv):
        raise TypeError("q and caches must share a dtype")
    B, Hq, d = qa.shape
    total, Hkv, dk_ = ka.shape
    if dk_ != d or va.shape != ka.shape:
        raise ValueError("shape mismatch between q and caches")
    cu = np.ascontiguousarray(np.asarray(torch.as_tensor(cu_seqlens).cpu(), dtype=np.int32))
    if cu.shape != (B + 1,) or (B > 0 and int(cu[-1]) > total):
        raise ValueError("cu_seqlens must have B+1 entries ending at most at the cache size")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    rb = np.ascontiguousarray(rows[:, 0].astype(np.int32))
    rh = np.ascontiguousarray(rows[:, 1].astype(np.int32))
    R = rows.shape[0]
    o = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros((R,), dtype=np.float64)
    rc = (lib or _load()).oracle_decode_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(cu), B, Hq, Hkv, d,
                                    float(scale), R, _ptr(rb), _ptr(rh), _ptr(o), _ptr(lse),
                                    _threads(nthreads))
    _check(rc)
    return o, lse


def decode(q, k_cache, v_cache, cu_seqlens, scale: float, nthreads: int = 0, lib=None):
    """Full decode.  Returns (o [B,Hq,d] float64, lse [B,Hq] float64)."""
    B, Hq, d = q.shape
    bb, hh = np.meshgrid(np.arange(B), np.arange(Hq), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel()], axis=1)
    o, lse = decode_rows(q, k_cache, v_cache, cu_seqlens, scale, rows, nthreads, lib)
    return o.reshape(B, Hq, d), lse.reshape(B, Hq)


def decode_append(q, k_cache, v_cache, cu_seqlens, k_new, v_new, scale: float, nthreads: int = 0, lib=None,
                  rows=None):
    """Decode after appending each sequence's new key/value row to its cache.

    The new token's key and value become row L_b of sequence b, after its L_b
    cached rows, and the token attends to all L_b + 1 rows (ai6s.net page,
    section "what ops-transformer adds", third item: the cache grows by one row
    per generated token and attention reads the cache's real length).  q
    [B,Hq,d]; k_cache/v_cache [total,Hkv,d] packed by cu_seqlens (host or
    device, int [B+1]); k_new/v_new [B,Hkv,d].  Returns (o [B,Hq,d], lse
    [B,Hq], k_after, v_after, cu_after): the decode result in float64 and the
    packed caches after the append (torch tensors of the caches' dtype).  With
    ``rows`` ((b, h) pairs, as for ``decode_rows``) o and lse are [R,d] and
    [R] for those pairs only.
    """
    cu = [int(x) for x in torch.as_tensor(cu_seqlens).cpu().tolist()]
    B = len(cu) - 1
    if k_new.shape[0] != B or v_new.shape != k_new.shape or k_new.shape[1:] != k_cache.shape[1:]:
        raise ValueError("k_new and v_new must be [B,Hkv,d] matching the caches")
    ks, vs, lens = [], [], []
    for b in range(B):
        ks += [k_cache[cu[b]:cu[b + 1]], k_new[b:b + 1]]
        vs += [v_cache[cu[b]:cu[b + 1]], v_new[b:b + 1]]
        lens.append(cu[b + 1] - cu[b] + 1)
    k_after = torch.cat(ks) if ks else k_cache[:0]
    v_after = torch.cat(vs) if vs else v_cache[:0]
    cu_after = torch.zeros(B + 1, dtype=torch.int32)
    cu_after[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    if rows is None:
        o, lse = decode(q, k_after, v_after, cu_after, scale, nthreads, lib)
    else:
        o, lse = decode_rows(q, k_after, v_after, cu_after, scale, rows, nthreads, lib)
    return o, lse, k_after, v_after, cu_after


def _f64(t) -> np.ndarray:
    """Exact float64 copy of a float64, float32 or bfloat16 tensor (bf16 and
    fp32 values are exactly representable in fp64)."""
    return torch.as_tensor(t).detach().cpu().to(torch.float64).numpy()


def attention_bwd(q, k, v, do, causal: bool, scale: float, kv_heads=None, with_magnitudes: bool = False):
    """Gradients of exact attention for a loss L with dL/dO = do.

    The pages give no backward algorithm (the training speed-ups on the
    effectstory.com page and the ai6s.net page's section "the data" rest on
    one); this is the derivative of the plain definition that the forward
    oracle computes (ai6s.net page, section "standard attention's fatal flaw is
    data movement, not compute": S = scale Q K^T, P = softmax(S) over the
    visible keys, O = P V), by the chain rule:
        dV = P^T dO,   dP = dO V^T,
        dS_ij = P_ij (dP_ij - sum_l P_il dP_il)       (the softmax Jacobian),
        dQ = scale dS K,   dK = scale dS^T Q,
    with the mask of the forward (bottom-right causal) and GQA heads summed
    into their kv head (kv head = h / (Hq/Hkv)).  A row with no visible key has
    P = 0 and contributes nothing.  Library matrix products in float64.

    q, do [B,N,Hq,d]; k, v [B,Nk,Hkv,d].  Returns (dq [B,N,Hq,d], dk, dv
    [B,Nk,Hkv,d]) in float64; with ``kv_heads`` (a list of kv heads) only those
    heads' dk, dv and their query heads' dq are computed (the rest are 0).
    With ``with_magnitudes`` it also returns (mq, mk, mv): the same sums with
    every term replaced by its absolute value (scale |dS| |K|, scale |dS|^T |Q|,
    P^T |dO|), plus, for dq and dk, the terms through which the row constant
    D_i = sum_l P_il dP_il enters dS (scale a_i P |K| and scale P^T (a |Q|),
    a_i = sum_d |dO_id O_id|); they bound the effect of rounding each term,
    and of computing D from a rounded O.
    """
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, Hq, d = Q.shape
    Nk, Hkv = K.shape[1], K.shape[2]
    if Hq % Hkv or dO.shape != Q.shape or V.shape != K.shape:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    dq, dk, dv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    mq, mk, mv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    visible = np.ones((N, Nk), dtype=bool)
    if causal:
        visible = np.arange(Nk)[None, :] <= np.arange(N)[:, None] + (Nk - N)
    for b in range(B):
        for g in (range(Hkv) if kv_heads is None else kv_heads):
            Kg, Vg = K[b, :, g, :], V[b, :, g, :]
            for h in range(g * G, (g + 1) * G):
                Qh, dOh = Q[b, :, h, :], dO[b, :, h, :]
                S = np.where(visible, scale * (Qh @ Kg.T), -np.inf)
                m = S.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                E = np.exp(S - m)                       # 0 where masked
                l = E.sum(axis=1, keepdims=True)
                P = np.divide(E, l, out=np.zeros_like(E), where=l > 0)
                dP = dOh @ Vg.T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dv[b, :, g, :] += P.T @ dOh
                dq[b, :, h, :] = scale * (dS @ Kg)
                dk[b, :, g, :] += scale * (dS.T @ Qh)
                if with_magnitudes:
                    aS = np.abs(dS)
                    a = np.abs(dOh * (P @ Vg)).sum(axis=1, keepdims=True)     # [N, 1]
                    mv[b, :, g, :] += P.T @ np.abs(dOh)
                    mq[b, :, h, :] = scale * ((aS + a * P) @ np.abs(Kg))
                    mk[b, :, g, :] += scale * ((aS + a * P).T @ np.abs(Qh))
    if with_magnitudes:
        return dq, dk, dv, (mq, mk, mv)
    return dq, dk, dv

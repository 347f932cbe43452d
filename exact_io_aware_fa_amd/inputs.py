"""Seeded synthetic inputs shared by the GPU path's tests, the benchmark and the
CPU oracle's tests.

This module holds no attention arithmetic: it only draws random numbers and
names the five workloads.  Every tensor is drawn on the CPU from a
``torch.Generator`` seeded with ``seed``: first the cache lengths (decode only),
then Q, K and V in that order as fp32 standard normals, each then rounded to the
storage dtype with ``Tensor.to`` (round to nearest even for bf16).  The GPU and
the oracle consume the same rounded tensors.

The shapes stand in for the workloads the pages measure (BERT-large at sequence
512 and GPT-2 at sequence 1K on the effectstory.com page's speed-up table;
Llama2-70B inference and the 32K sequence limit on the ai6s.net page, section
"the data"); no dataset or weight is used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


def fp32_scale(d: int) -> float:
    """The softmax scale 1/sqrt(d) as the fp32 value handed to every path."""
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    N: int
    Nk: int
    d: int
    causal: bool

    @property
    def scale(self) -> float:
        return fp32_scale(self.d)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int          # inclusive
    len_hi: int          # inclusive

    @property
    def scale(self) -> float:
        return fp32_scale(self.d)


# The five workloads, in order.
SINGLE_HEAD_F32 = PrefillConfig("single-head fp32 B1 H1 N256 d64", torch.float32,
                                1, 1, 1, 256, 256, 64, False)
BERT_LARGE_BF16 = PrefillConfig("BERT-large-shaped bf16 B16 H16 N512 d64", torch.bfloat16,
                                16, 16, 16, 512, 512, 64, False)
GPT2_CAUSAL_BF16 = PrefillConfig("GPT-2-shaped causal bf16 B8 H12 N1024 d64", torch.bfloat16,
                                 8, 12, 12, 1024, 1024, 64, True)
LLAMA70B_GQA_BF16 = PrefillConfig("Llama2-70B-shaped causal GQA bf16 B1 Hq64 Hkv8 N8192 d128",
                                  torch.bfloat16, 1, 64, 8, 8192, 8192, 128, True)
DECODE_VARLEN_BF16 = DecodeConfig("varlen KV-cache decode bf16 32 seqs L512-32768 Hq64 Hkv8 d128",
                                  torch.bfloat16, 32, 64, 8, 128, 512, 32768)

PREFILL_CONFIGS = (SINGLE_HEAD_F32, BERT_LARGE_BF16, GPT2_CAUSAL_BF16, LLAMA70B_GQA_BF16)


@dataclass(frozen=True)
class VarlenConfig:
    """Chunked prefill: B sequences, each a chunk of `chunk` new query tokens
    appended to a cache of ctx_lo..ctx_hi (inclusive, uniform) earlier tokens,
    so N_b = chunk and Nk_b = ctx_b + chunk."""
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    chunk: int
    ctx_lo: int
    ctx_hi: int

    @property
    def scale(self) -> float:
        return fp32_scale(self.d)


# Llama2-70B-shaped heads; chunks and cache lengths up to the 16K context the
# pages' Llama2-70B discussion works within (ai6s.net page, section "the data").
VARLEN_CHUNKED_BF16 = VarlenConfig("chunked prefill bf16 16 seqs: 2048-token chunks on 0-14336 cached tokens, "
                                   "Hq64 Hkv8 d128, causal", torch.bfloat16, 16, 64, 8, 128, True, 2048, 0, 14336)


def _normal(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def prefill_inputs(B: int, N: int, Nk: int, Hq: int, Hkv: int, d: int,
                   dtype: torch.dtype = torch.bfloat16, seed: int = 0, q_mult: float = 1.0):
    """Q [B,N,Hq,d], K and V [B,Nk,Hkv,d] on the CPU (BSHD, contiguous).

    ``q_mult`` scales the fp32 draw of Q before rounding (a stress option for
    peaked softmax rows); it is 1 for every named workload.
    """
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, N, Hq, d), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q = q * q_mult
    q = q.to(dtype)
    k = _normal(g, (B, Nk, Hkv, d), dtype)
    v = _normal(g, (B, Nk, Hkv, d), dtype)
    return q, k, v


def prefill_config_inputs(cfg: PrefillConfig, seed: int = 0):
    return prefill_inputs(cfg.B, cfg.N, cfg.Nk, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, seed)


def decode_lengths(B: int, lo: int, hi: int, g: torch.Generator) -> torch.Tensor:
    """B cache lengths uniform on the integers lo..hi inclusive (int64, CPU)."""
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)


def cu_from_lengths(lens) -> torch.Tensor:
    """int32 [B+1] prefix offsets of a packed cache (cu[0] = 0)."""
    lens = torch.as_tensor(lens, dtype=torch.int64)
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    return cu.to(torch.int32)


def decode_inputs(lens, Hq: int, Hkv: int, d: int, dtype: torch.dtype = torch.bfloat16,
                  seed: int = 0, g: torch.Generator | None = None):
    """Q [B,Hq,d], packed K/V caches [sum(lens),Hkv,d] and cu_seqlens int32 [B+1]."""
    if g is None:
        g = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(lens, dtype=torch.int64)
    B = lens.numel()
    total = int(lens.sum())
    q = _normal(g, (B, Hq, d), dtype)
    kc = _normal(g, (total, Hkv, d), dtype)
    vc = _normal(g, (total, Hkv, d), dtype)
    return q, kc, vc, cu_from_lengths(lens)


def decode_config_inputs(cfg: DecodeConfig, seed: int = 0):
    """Lengths are drawn first from the same generator, then Q, K, V."""
    g = torch.Generator().manual_seed(seed)
    lens = decode_lengths(cfg.B, cfg.len_lo, cfg.len_hi, g)
    q, kc, vc, cu = decode_inputs(lens, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, g=g)
    return q, kc, vc, cu, lens


def varlen_inputs(q_lens, k_lens, Hq: int, Hkv: int, d: int, dtype: torch.dtype = torch.bfloat16,
                  seed: int = 0, g: torch.Generator | None = None):
    """Packed Q [sum(q_lens),Hq,d], K/V [sum(k_lens),Hkv,d] and cu_seqlens_q/k int32 [B+1]."""
    if g is None:
        g = torch.Generator().manual_seed(seed)
    q_lens = torch.as_tensor(q_lens, dtype=torch.int64)
    k_lens = torch.as_tensor(k_lens, dtype=torch.int64)
    q = _normal(g, (int(q_lens.sum()), Hq, d), dtype)
    k = _normal(g, (int(k_lens.sum()), Hkv, d), dtype)
    v = _normal(g, (int(k_lens.sum()), Hkv, d), dtype)
    return q, k, v, cu_from_lengths(q_lens), cu_from_lengths(k_lens)


def varlen_config_inputs(cfg: VarlenConfig, seed: int = 0):
    """The cached lengths are drawn first from the same generator, then Q, K, V."""
    g = torch.Generator().manual_seed(seed)
    ctx = torch.randint(cfg.ctx_lo, cfg.ctx_hi + 1, (cfg.B,), generator=g, dtype=torch.int64)
    q_lens = torch.full((cfg.B,), cfg.chunk, dtype=torch.int64)
    k_lens = ctx + cfg.chunk
    q, k, v, cu_q, cu_k = varlen_inputs(q_lens, k_lens, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, g=g)
    return q, k, v, cu_q, cu_k, q_lens, k_lens


def paged_decode_inputs(lens, Hq: int, Hkv: int, d: int, block_size: int, dtype: torch.dtype = torch.bfloat16,
                        seed: int = 0, g: torch.Generator | None = None, spare_blocks: int = 3,
                        fill: float = float("nan")):
    """A decode step on a paged KV cache with one new row per sequence.

    Draws, in order: Q, the packed caches K and V (as ``decode_inputs``), the
    new rows k_new and v_new [B,Hkv,d], and a random order of the physical
    blocks.  Sequence b gets ceil((L_b + 1) / block_size) blocks (room for the
    new row), taken in that random order; its logical row i sits in row
    i % block_size of block block_table[b, i // block_size].  Page rows that
    hold no cached row are ``fill`` (NaN by default, so that a read of one
    shows in the result).  Returns a dict with the packed view (q, kc, vc, cu),
    the new rows, the pages k_pages/v_pages [num_blocks, block_size, Hkv, d],
    block_table int32 [B, max_blocks] (unused entries -1) and seqlens int32 [B].
    """
    if g is None:
        g = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(lens, dtype=torch.int64)
    q, kc, vc, cu = decode_inputs(lens, Hq, Hkv, d, dtype, g=g)
    B = lens.numel()
    k_new = _normal(g, (B, Hkv, d), dtype)
    v_new = _normal(g, (B, Hkv, d), dtype)
    need = [(int(L) + 1 + block_size - 1) // block_size for L in lens.tolist()]
    num_blocks = sum(need) + spare_blocks
    order = torch.randperm(num_blocks, generator=g)
    max_blocks = max(need) + 1 if need else 1
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    k_pages = torch.full((num_blocks, block_size, Hkv, d), fill, dtype=dtype)
    v_pages = torch.full((num_blocks, block_size, Hkv, d), fill, dtype=dtype)
    nxt = 0
    for b in range(B):
        L, s = int(lens[b]), int(cu[b])
        for i in range(need[b]):
            pb = int(order[nxt])
            nxt += 1
            table[b, i] = pb
            r0, r1 = i * block_size, min(L, (i + 1) * block_size)
            if r1 > r0:
                k_pages[pb, :r1 - r0] = kc[s + r0:s + r1]
                v_pages[pb, :r1 - r0] = vc[s + r0:s + r1]
    return {"q": q, "kc": kc, "vc": vc, "cu": cu, "k_new": k_new, "v_new": v_new, "k_pages": k_pages,
            "v_pages": v_pages, "block_table": table, "seqlens": lens.to(torch.int32)}


def paged_config_inputs(cfg: DecodeConfig, block_size: int, seed: int = 0, fill: float = 0.0):
    """The decode workload on a paged cache: the same lengths, Q, K and V as
    ``decode_config_inputs`` (drawn first, in that order), then the new rows
    and the block order."""
    g = torch.Generator().manual_seed(seed)
    lens = decode_lengths(cfg.B, cfg.len_lo, cfg.len_hi, g)
    return paged_decode_inputs(lens, cfg.Hq, cfg.Hkv, cfg.d, block_size, cfg.dtype, g=g, fill=fill)

"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible mistake in the oracle (a dropped scale,
a wrong mask sign or offset, a transposed operand, the wrong kv head, a base-2
LSE, a missing normalisation) fails at least one of them; ``test_oracle_mutants``
plants such mistakes in copies of the oracle source and checks exactly that.

Sources of the facts pinned: the definition of exact attention (ai6s.net page,
sections "standard attention's fatal flaw is data movement, not compute" and
"FlashAttention changes the dataflow, not the algorithm"); the causal mask and
variable-length cache (same page, section "what ops-transformer adds", second
and third items).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle
from tests import brute
from exact_io_aware_fa_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
_MATH = {"log": math.log, "exp": math.exp, "sqrt": math.sqrt, "inf": math.inf}


def _val(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, _MATH))
    return float(x)


def _arr(nested):
    return np.vectorize(_val, otypes=[np.float64])(np.array(nested, dtype=object))


def _close(a, b, tol):
    """Elementwise |a-b| <= tol, with equal infinities counted as equal."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert not np.isnan(a).any() and not np.isnan(b).any()
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    assert err.max(initial=0.0) <= tol, "max abs err %g > %g" % (err.max(), tol)


def _randn(g, *shape):
    return torch.randn(shape, generator=g, dtype=torch.float64)


# --------------------------------------------------------------- worked examples

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["prefill"], ids=lambda c: c["name"])
def test_golden_prefill(case):
    q = torch.from_numpy(_arr(case["q"]))
    k = torch.from_numpy(_arr(case["k"]))
    v = torch.from_numpy(_arr(case["v"]))
    o, lse = oracle.attention(q, k, v, case["causal"], case["scale"])
    _close(o, _arr(case["o"]), 1e-12)
    _close(lse, _arr(case["lse"]), 1e-12)


@pytest.mark.parametrize("case", _golden()["decode"], ids=lambda c: c["name"])
def test_golden_decode(case):
    q = torch.from_numpy(_arr(case["q"]))
    kc = torch.from_numpy(_arr(case["k_cache"]))
    vc = torch.from_numpy(_arr(case["v_cache"]))
    cu = torch.tensor(case["cu_seqlens"], dtype=torch.int32)
    o, lse = oracle.decode(q, kc, vc, cu, case["scale"])
    _close(o, _arr(case["o"]), 1e-12)
    _close(lse, _arr(case["lse"]), 1e-12)


# ------------------------------------------------------------------ brute force

BRUTE_SHAPES = [
    # (Hq, Hkv, N, Nk, d)
    (1, 1, 1, 1, 4), (1, 1, 2, 3, 4), (2, 1, 3, 2, 4), (4, 2, 17, 17, 4),
    (4, 1, 3, 17, 4), (2, 2, 17, 3, 4), (1, 1, 5, 5, 64), (4, 2, 2, 17, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", BRUTE_SHAPES)
def test_brute_force_tiny(shape, causal):
    Hq, Hkv, N, Nk, d = shape
    g = torch.Generator().manual_seed(hash(shape) % 1000 + causal)
    q, k, v = _randn(g, 1, N, Hq, d), _randn(g, 1, Nk, Hkv, d), _randn(g, 1, Nk, Hkv, d)
    scale = inputs.fp32_scale(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    bo, blse = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    _close(o, bo, 1e-12)
    _close(lse, blse, 1e-12)


# ------------------------------------------------- variable-length prefill

VARLEN_TINY = [
    # (q_lens, k_lens): chunks shorter than their caches, an empty chunk, a
    # chunk with no cache rows, single rows
    ((3, 0, 2, 1, 4), (5, 4, 0, 1, 4)),
    ((1, 6), (9, 6)),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", VARLEN_TINY)
def test_varlen_brute_force_tiny(lens, causal):
    """Each packed sequence equals the brute force of that sequence alone
    (bottom-right causal within the sequence), in the [total_q,Hq,d] / [Hq,total_q] layouts."""
    q_lens, k_lens = lens
    Hq, Hkv, d = 4, 2, 4
    q, k, v, cu_q, cu_k = inputs.varlen_inputs(q_lens, k_lens, Hq, Hkv, d, torch.float64, seed=len(q_lens) + causal)
    scale = inputs.fp32_scale(d)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale)
    cq, ck = cu_q.tolist(), cu_k.tolist()
    for b in range(len(q_lens)):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe == qs:
            continue
        if ke == ks:        # no keys: O = 0, LSE = -inf
            assert np.all(o[qs:qe] == 0.0) and np.all(lse[:, qs:qe] == -math.inf)
            continue
        bo, blse = brute.attention([q[qs:qe].tolist()], [k[ks:ke].tolist()], [v[ks:ke].tolist()], causal, scale)
        _close(o[qs:qe], np.asarray(bo[0]), 1e-12)
        _close(lse[:, qs:qe], np.asarray(blse[0]), 1e-12)


def test_varlen_equal_lengths_match_batched():
    """Packing B equal-length sequences gives the batched [B,N,H,d] result, with
    LSE [B,Hq,N] laid out as [Hq, B*N]."""
    B, N, Nk, Hq, Hkv, d = 3, 5, 9, 4, 2, 8
    g = torch.Generator().manual_seed(11)
    q, k, v = _randn(g, B, N, Hq, d), _randn(g, B, Nk, Hkv, d), _randn(g, B, Nk, Hkv, d)
    scale = inputs.fp32_scale(d)
    for causal in (False, True):
        ro, rl = oracle.attention(q, k, v, causal, scale)
        o, lse = oracle.attention_varlen(q.reshape(B * N, Hq, d), k.reshape(B * Nk, Hkv, d),
                                         v.reshape(B * Nk, Hkv, d), inputs.cu_from_lengths([N] * B),
                                         inputs.cu_from_lengths([Nk] * B), causal, scale)
        _close(o, ro.reshape(B * N, Hq, d), 0.0)
        _close(lse, rl.transpose(1, 0, 2).reshape(Hq, B * N), 0.0)


def test_varlen_other_sequences_have_no_effect():
    q, k, v, cu_q, cu_k = inputs.varlen_inputs((4, 3), (6, 5), 2, 1, 8, torch.float64, seed=3)
    scale = inputs.fp32_scale(8)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, True, scale)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:4] *= 7.0
    k2[:6] += 3.0
    v2[:6] -= 5.0
    o2, lse2 = oracle.attention_varlen(q2, k2, v2, cu_q, cu_k, True, scale)
    assert np.array_equal(o[4:], o2[4:]) and np.array_equal(lse[:, 4:], lse2[:, 4:])
    assert not np.array_equal(o[:4], o2[:4])


# ------------------------------------------------- reduction to library routines

@pytest.mark.parametrize("Hq,Hkv,N,d", [(4, 4, 33, 16), (8, 2, 40, 64), (6, 3, 65, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(Hq, Hkv, N, d, causal):
    """torch SDPA in fp64 on the CPU (square case, where its top-left causal mask
    equals bottom-right) and torch.logsumexp over a torch.tril mask."""
    g = torch.Generator().manual_seed(N * 7 + d + causal)
    B = 2
    q, k, v = _randn(g, B, N, Hq, d), _randn(g, B, N, Hkv, d), _randn(g, B, N, Hkv, d)
    scale = inputs.fp32_scale(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    qh = q.transpose(1, 2)
    kh = k.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    vh = v.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    ref = F.scaled_dot_product_attention(qh, kh, vh, is_causal=causal, scale=scale)
    _close(o, ref.transpose(1, 2).numpy(), 1e-12)
    s = torch.matmul(qh, kh.transpose(-1, -2)) * scale
    if causal:
        keep = torch.ones(N, N, dtype=torch.bool).tril()
        s = s.masked_fill(~keep, -math.inf)
    _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12)


def test_bf16_workload_slice_matches_sdpa():
    """A slice of the BERT-large-shaped bf16 workload, widened exactly."""
    cfg = inputs.BERT_LARGE_BF16
    q, k, v = inputs.prefill_config_inputs(cfg)
    q, k, v = q[:1, :, :2], k[:1, :, :2], v[:1, :, :2]
    o, lse = oracle.attention(q, k, v, False, cfg.scale)
    ref = F.scaled_dot_product_attention(q.double().transpose(1, 2), k.double().transpose(1, 2),
                                         v.double().transpose(1, 2), scale=cfg.scale)
    _close(o, ref.transpose(1, 2).numpy(), 1e-12)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("N,Nk,causal", [(5, 5, False), (5, 5, True), (3, 9, True), (9, 4, True)])
def test_identical_keys_average_visible_values(N, Nk, causal):
    """All keys equal: the softmax is uniform over the visible keys, so O_i is the
    mean of the visible V rows and LSE_i = scale*q_i.k + ln(#visible)."""
    g = torch.Generator().manual_seed(11)
    d, Hq = 8, 2
    q = _randn(g, 1, N, Hq, d)
    krow = _randn(g, d)
    k = krow.expand(1, Nk, 1, d).contiguous()
    v = _randn(g, 1, Nk, 1, d)
    scale = 0.3
    o, lse = oracle.attention(q, k, v, causal, scale)
    for i in range(N):
        nvis = min(Nk, i + Nk - N + 1) if causal else Nk
        for h in range(Hq):
            if nvis <= 0:
                assert np.all(o[0, i, h] == 0.0) and lse[0, h, i] == -math.inf
                continue
            mean_v = v[0, :nvis, 0].mean(dim=0).numpy()
            _close(o[0, i, h], mean_v, 1e-12)
            expect = scale * float(q[0, i, h] @ krow) + math.log(nvis)
            _close(lse[0, h, i], expect, 1e-12)


def test_single_key_returns_v_exactly():
    """Nk = 1: the only weight is exp(0)/1 = 1, so O = V[0] bit for bit and LSE = scale*q.k."""
    g = torch.Generator().manual_seed(5)
    q, k, v = _randn(g, 2, 7, 4, 16), _randn(g, 2, 1, 2, 16), _randn(g, 2, 1, 2, 16)
    o, lse = oracle.attention(q, k, v, False, 0.25)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, :, h], v[b, 0, h // 2].expand(7, 16).numpy())
            _close(lse[b, h], (0.25 * (q[b, :, h] @ k[b, 0, h // 2])).numpy(), 1e-13)


def test_zero_queries_count_visible_keys():
    """Q = 0 makes every visible score 0, so LSE_i = ln(count of visible keys):
    bottom-right causal gives i + 1 + Nk - N, non-causal gives Nk."""
    B, Hq, Hkv, d = 1, 2, 1, 8
    for N, Nk in [(7, 7), (4, 11), (1, 33)]:
        g = torch.Generator().manual_seed(N + Nk)
        q = torch.zeros(B, N, Hq, d, dtype=torch.float64)
        k, v = _randn(g, B, Nk, Hkv, d), _randn(g, B, Nk, Hkv, d)
        _, lse_c = oracle.attention(q, k, v, True, 0.125)
        _, lse_n = oracle.attention(q, k, v, False, 0.125)
        for i in range(N):
            _close(lse_c[0, :, i], [math.log(i + 1 + Nk - N)] * Hq, 1e-12)
            _close(lse_n[0, :, i], [math.log(Nk)] * Hq, 1e-12)


# ------------------------------------------------------------------ invariances

def test_permuting_keys_and_values_together():
    g = torch.Generator().manual_seed(3)
    q, k, v = _randn(g, 2, 9, 4, 32), _randn(g, 2, 23, 2, 32), _randn(g, 2, 23, 2, 32)
    perm = torch.randperm(23, generator=g)
    o1, l1 = oracle.attention(q, k, v, False, 0.2)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], False, 0.2)
    _close(o1, o2, 1e-12)
    _close(l1, l2, 1e-12)


def test_linear_in_values():
    g = torch.Generator().manual_seed(4)
    q, k = _randn(g, 1, 12, 2, 16), _randn(g, 1, 12, 2, 16)
    v1, v2 = _randn(g, 1, 12, 2, 16), _randn(g, 1, 12, 2, 16)
    a, b = 0.75, -2.5
    for causal in (False, True):
        o1, _ = oracle.attention(q, k, v1, causal, 0.25)
        o2, _ = oracle.attention(q, k, v2, causal, 0.25)
        o3, _ = oracle.attention(q, k, a * v1 + b * v2, causal, 0.25)
        _close(o3, a * o1 + b * o2, 1e-12)


def test_shifting_all_keys_shifts_lse_only():
    """k_j -> k_j + u adds scale*q.u to every score of the row: O unchanged,
    LSE shifted by scale*q.u."""
    g = torch.Generator().manual_seed(6)
    q, k, v = _randn(g, 1, 10, 3, 16), _randn(g, 1, 14, 3, 16), _randn(g, 1, 14, 3, 16)
    u = _randn(g, 16)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal, 0.5)
        o2, l2 = oracle.attention(q, k + u, v, causal, 0.5)
        _close(o1, o2, 1e-12)
        shift = (0.5 * (q[0] @ u)).transpose(0, 1).numpy()      # [Hq, N]
        _close(l2[0], l1[0] + shift, 1e-12)


def test_gqa_equals_repeated_kv_heads():
    """Grouped heads read kv head h // (Hq/Hkv): the same as repeat_interleave."""
    g = torch.Generator().manual_seed(8)
    q, k, v = _randn(g, 2, 6, 8, 16), _randn(g, 2, 6, 2, 16), _randn(g, 2, 6, 2, 16)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal, 0.25)
        o2, l2 = oracle.attention(q, k.repeat_interleave(4, dim=2),
                                  v.repeat_interleave(4, dim=2), causal, 0.25)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_bottom_right_causal_rows_are_prefix_attention():
    """With N < Nk, causal row i equals non-causal attention over keys
    0 .. i + Nk - N, and equals the matching row of the square causal problem
    whose extra leading queries are arbitrary."""
    g = torch.Generator().manual_seed(9)
    N, Nk, Hq, d = 5, 12, 2, 16
    q, k, v = _randn(g, 1, N, Hq, d), _randn(g, 1, Nk, Hq, d), _randn(g, 1, Nk, Hq, d)
    o, lse = oracle.attention(q, k, v, True, 0.25)
    for i in range(N):
        last = i + Nk - N
        op, lp = oracle.attention(q[:, i:i + 1], k[:, :last + 1], v[:, :last + 1], False, 0.25)
        _close(o[:, i], op[:, 0], 1e-12)
        _close(lse[:, :, i], lp[:, :, 0], 1e-12)
    qsq = torch.cat([_randn(g, 1, Nk - N, Hq, d), q], dim=1)
    osq, lsq = oracle.attention(qsq, k, v, True, 0.25)
    _close(o, osq[:, Nk - N:], 1e-12)
    _close(lse, lsq[:, :, Nk - N:], 1e-12)


def test_rows_sum_to_one_is_enforced():
    """The oracle asserts |sum_j P_ij - 1| <= 1e-12 per row; normal inputs pass,
    including very peaked rows (large scale)."""
    g = torch.Generator().manual_seed(10)
    q, k, v = _randn(g, 1, 8, 1, 8), _randn(g, 1, 8, 1, 8), _randn(g, 1, 8, 1, 8)
    oracle.attention(q, k, v, False, 50.0)


# --------------------------------------------------------------------- decode

def test_decode_equals_single_row_prefill():
    lens = [1, 7, 33, 0, 20]
    q, kc, vc, cu = inputs.decode_inputs(lens, 8, 2, 16, torch.float32, seed=2)
    o, lse = oracle.decode(q, kc, vc, cu, 0.25)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o[b] == 0.0) and np.all(lse[b] == -math.inf)
            continue
        s, e = int(cu[b]), int(cu[b + 1])
        op, lp = oracle.attention(q[b:b + 1, None], kc[None, s:e], vc[None, s:e], False, 0.25)
        assert np.array_equal(o[b], op[0, 0]) and np.array_equal(lse[b], lp[0, :, 0])


def test_decode_matches_torch_sdpa_and_ignores_other_sequences():
    lens = [3, 17, 9]
    q, kc, vc, cu = inputs.decode_inputs(lens, 4, 2, 32, torch.float64, seed=3)
    o, lse = oracle.decode(q, kc, vc, cu, 0.2)
    for b in range(3):
        s, e = int(cu[b]), int(cu[b + 1])
        kh = kc[s:e].transpose(0, 1).repeat_interleave(2, dim=0)     # [Hq, L, d]
        vh = vc[s:e].transpose(0, 1).repeat_interleave(2, dim=0)
        ref = F.scaled_dot_product_attention(q[b][:, None], kh, vh, scale=0.2)[:, 0]
        _close(o[b], ref.numpy(), 1e-12)
        _close(lse[b], torch.logsumexp(0.2 * (kh @ q[b][:, :, None])[..., 0], -1).numpy(), 1e-12)
    # rows belonging to other sequences have no effect, bit for bit
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[cu[1]:cu[2]] = _randn(torch.Generator().manual_seed(0), lens[1], 2, 32)
    vc2[cu[1]:cu[2]] = 7.0
    o2, lse2 = oracle.decode(q, kc2, vc2, cu, 0.2)
    for b in (0, 2):
        assert np.array_equal(o[b], o2[b]) and np.array_equal(lse[b], lse2[b])


def _new_rows(B, Hkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return _randn(g, B, Hkv, d).to(dtype), _randn(g, B, Hkv, d).to(dtype)


def test_decode_append_brute_force_tiny():
    """Each token attends to its cached rows plus its own new row, checked by the
    scalar brute force; an empty cache leaves only the new row."""
    lens = [0, 1, 5, 3]
    Hq, Hkv, d, scale = 4, 2, 8, 0.3
    q, kc, vc, cu = inputs.decode_inputs(lens, Hq, Hkv, d, torch.float64, seed=11)
    kn, vn = _new_rows(len(lens), Hkv, d, torch.float64, 12)
    o, lse, ka, va, cua = oracle.decode_append(q, kc, vc, cu, kn, vn, scale)
    for b, L in enumerate(lens):
        s = int(cu[b])
        keys = torch.cat([kc[s:s + L], kn[b:b + 1]])
        vals = torch.cat([vc[s:s + L], vn[b:b + 1]])
        bo, bl = brute.attention([[q[b].tolist()]], [keys.tolist()], [vals.tolist()], False, scale)
        _close(o[b], np.array(bo[0][0]), 1e-12)
        _close(lse[b], np.array([bl[0][h][0] for h in range(Hq)]), 1e-12)
    # the caches after the append: each sequence's rows, then its new row
    assert [int(x) for x in cua] == [0, 1, 3, 9, 13]
    assert torch.equal(ka[cua[1] - 1], kn[0]) and torch.equal(va[cua[3] - 1], vn[2])
    assert torch.equal(ka[cua[2]:cua[3] - 1], kc[cu[2]:cu[3]])


def test_decode_append_to_empty_cache_returns_new_value_exactly():
    """A single visible key: O = v_new exactly and LSE = scale * q . k_new."""
    q, kc, vc, cu = inputs.decode_inputs([0, 0], 2, 1, 16, torch.float64, seed=13)
    kn, vn = _new_rows(2, 1, 16, torch.float64, 14)
    o, lse, _, _, _ = oracle.decode_append(q, kc, vc, cu, kn, vn, 0.25)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(o[b, h], vn[b, 0].numpy())
            assert abs(lse[b, h] - 0.25 * math.fsum((q[b, h] * kn[b, 0]).tolist())) <= 1e-13


def test_decode_append_merges_with_the_cached_result():
    """Appending one key merges the cached result with the new row by the
    logsumexp identity: LSE' = log(exp(LSE) + exp(s)), O' = w O + (1 - w) v_new
    with w = exp(LSE - LSE'), s = scale * q . k_new (two oracle calls related
    by the rescaling identity the online softmax rests on)."""
    lens = [6, 40, 1]
    Hq, Hkv, d, scale = 8, 2, 32, 0.17
    q, kc, vc, cu = inputs.decode_inputs(lens, Hq, Hkv, d, torch.float64, seed=15)
    kn, vn = _new_rows(3, Hkv, d, torch.float64, 16)
    o0, l0 = oracle.decode(q, kc, vc, cu, scale)
    o1, l1, _, _, _ = oracle.decode_append(q, kc, vc, cu, kn, vn, scale)
    G = Hq // Hkv
    for b in range(3):
        for h in range(Hq):
            s = scale * math.fsum((q[b, h] * kn[b, h // G]).tolist())
            lse_new = max(l0[b, h], s) + math.log1p(math.exp(-abs(l0[b, h] - s)))
            w = math.exp(l0[b, h] - lse_new)
            assert abs(l1[b, h] - lse_new) <= 1e-12
            _close(o1[b, h], w * o0[b, h] + (1 - w) * vn[b, h // G].numpy(), 1e-12)


def test_decode_append_dominant_new_key_selects_new_value():
    """A new key whose score exceeds every cached one by far more than the fp64
    range takes all the weight: O = v_new, whichever cached rows precede it."""
    lens = [9, 2]
    q, kc, vc, cu = inputs.decode_inputs(lens, 2, 1, 4, torch.float64, seed=17)
    q[:, :, :] = torch.tensor([1.0, 0.0, 0.0, 0.0], dtype=torch.float64)
    kc[:, :, 0] = 0.0                                    # cached scores are 0
    kn = torch.zeros(2, 1, 4, dtype=torch.float64)
    kn[:, 0, 0] = 2000.0                                 # new score 2000 * scale
    _, vn = _new_rows(2, 1, 4, torch.float64, 18)
    o, lse, _, _, _ = oracle.decode_append(q, kc, vc, cu, kn, vn, 1.0)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(o[b, h], vn[b, 0].numpy())
            assert lse[b, h] == 2000.0


# ----------------------------------------------------------- input handling

def test_bf16_inputs_are_widened_exactly():
    q, k, v = inputs.prefill_inputs(1, 9, 9, 2, 1, 64, torch.bfloat16, seed=1)
    o1, l1 = oracle.attention(q, k, v, True, 0.125)
    o2, l2 = oracle.attention(q.double(), k.double(), v.double(), True, 0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_result_independent_of_thread_count():
    q, k, v = inputs.prefill_inputs(2, 40, 40, 4, 2, 32, torch.float32, seed=4)
    o1, l1 = oracle.attention(q, k, v, True, 0.2, nthreads=1)
    o2, l2 = oracle.attention(q, k, v, True, 0.2, nthreads=7)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_sampling_matches_full_run():
    q, k, v = inputs.prefill_inputs(2, 30, 30, 4, 2, 32, torch.bfloat16, seed=5)
    o, lse = oracle.attention(q, k, v, True, 0.125)
    rows = np.array([[1, 3, 29], [0, 0, 0], [1, 1, 17]])
    orow, lrow = oracle.attention_rows(q, k, v, True, 0.125, rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[r], o[b, i, h]) and lrow[r] == lse[b, h, i]


def test_invalid_arguments_raise():
    q, k, v = inputs.prefill_inputs(1, 4, 4, 3, 2, 8, torch.float32)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, v, False, 0.1)             # Hq % Hkv != 0
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q[:, :, :2], k, v, False, 0.1, [[0, 0, 4]])   # row out of range


def test_workload_recipe_decode_lengths():
    """Seed 0 draws the decode lengths first, uniform on 512..32768 inclusive."""
    g = torch.Generator().manual_seed(0)
    lens = inputs.decode_lengths(32, 512, 32768, g)
    assert lens.numel() == 32 and int(lens.min()) >= 512 and int(lens.max()) <= 32768
    cu = inputs.cu_from_lengths(lens)
    assert cu.dtype == torch.int32 and int(cu[0]) == 0 and int(cu[-1]) == int(lens.sum())

"""Pins of the backward oracle (``oracle.attention_bwd``) against things other
than itself (CPU only): central finite differences of the pinned forward
oracle, torch autograd through SDPA in float64, closed forms, and the GQA
reduction.  The gradients are those of the exact-attention definition (ai6s.net
page, section "standard attention's fatal flaw is data movement, not compute";
causal mask from section "what ops-transformer adds", second item).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from exact_io_aware_fa_amd import inputs
from oracle import oracle
from tests import brute


def _rand(shape, seed):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed), dtype=torch.float64)


@pytest.mark.parametrize("N,Nk,causal", [(3, 5, False), (3, 5, True), (5, 3, True), (4, 4, True)])
def test_bwd_matches_central_differences_of_the_forward(N, Nk, causal):
    """dL/dx for L = sum(O * dO), every element of q, k and v, by central
    differences of the forward oracle (step 1e-5: truncation ~1e-10)."""
    B, Hq, Hkv, d, scale = 1, 2, 1, 4, 0.7
    q, k, v = inputs.prefill_inputs(B, N, Nk, Hq, Hkv, d, torch.float64, seed=N * 10 + Nk)
    do = _rand(q.shape, 3)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, causal, scale)
        return float((o * do.numpy()).sum())

    eps = 1e-5
    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros(t.shape)
        for idx in np.ndindex(*t.shape):
            tp, tm = t.clone(), t.clone()
            tp[idx] += eps
            tm[idx] -= eps
            args_p = {"q": (tp, k, v), "k": (q, tp, v), "v": (q, k, tp)}[name]
            args_m = {"q": (tm, k, v), "k": (q, tm, v), "v": (q, k, tm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.abs(num - grad).max() <= 1e-7, name


@pytest.mark.parametrize("Hq,Hkv,N,causal", [(4, 2, 16, False), (4, 2, 16, True), (6, 3, 9, False), (2, 2, 7, True)])
def test_bwd_matches_torch_autograd_of_sdpa(Hq, Hkv, N, causal):
    """Reduction to a library routine: torch's SDPA in float64 with autograd
    (causal only where N = Nk, since SDPA's mask is top-left)."""
    d, scale = 16, 0.25
    q, k, v = inputs.prefill_inputs(2, N, N, Hq, Hkv, d, torch.float64, seed=Hq + N)
    do = _rand(q.shape, 5)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale)
    qt = q.transpose(1, 2).clone().requires_grad_(True)
    kt = k.transpose(1, 2).clone().requires_grad_(True)
    vt = v.transpose(1, 2).clone().requires_grad_(True)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale, enable_gqa=True)
    o.backward(do.transpose(1, 2))
    assert np.abs(qt.grad.transpose(1, 2).numpy() - dq).max() <= 1e-12
    assert np.abs(kt.grad.transpose(1, 2).numpy() - dk).max() <= 1e-12
    assert np.abs(vt.grad.transpose(1, 2).numpy() - dv).max() <= 1e-12


def test_bwd_single_key_closed_form():
    """With one key, O = v_0 whatever q and k are: dq = dk = 0 exactly and dv is
    the sum of dO over the group's query rows and heads."""
    q, k, v = inputs.prefill_inputs(1, 6, 1, 4, 2, 8, torch.float64, seed=7)
    do = _rand(q.shape, 8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, False, 0.5)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    ref = do.numpy().reshape(1, 6, 2, 2, 8).sum(axis=(1, 3))      # [B, Hkv, d]
    assert np.abs(dv[:, 0] - ref).max() <= 1e-13


def test_bwd_rows_without_keys_contribute_nothing():
    """Causal with N > Nk: the leading N - Nk rows see no key; their dq is 0 and
    changing their dO leaves dk and dv unchanged."""
    q, k, v = inputs.prefill_inputs(1, 9, 4, 2, 1, 8, torch.float64, seed=9)
    do = _rand(q.shape, 10)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, True, 0.4)
    assert np.all(dq[:, :5] == 0.0)
    do2 = do.clone()
    do2[:, :5] = 100.0
    _, dk2, dv2 = oracle.attention_bwd(q, k, v, do2, True, 0.4)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_bwd_gqa_sums_the_repeated_heads():
    """GQA gradients of a kv head are the sums over its query heads of the MHA
    gradients with K/V repeated per query head."""
    q, k, v = inputs.prefill_inputs(1, 11, 13, 6, 2, 8, torch.float64, seed=12)
    do = _rand(q.shape, 13)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, True, 0.3)
    kr, vr = k.repeat_interleave(3, dim=2), v.repeat_interleave(3, dim=2)
    dq_m, dk_m, dv_m = oracle.attention_bwd(q, kr, vr, do, True, 0.3)
    assert np.abs(dq - dq_m).max() <= 1e-13
    assert np.abs(dk - dk_m.reshape(1, 13, 2, 3, 8).sum(axis=3)).max() <= 1e-13
    assert np.abs(dv - dv_m.reshape(1, 13, 2, 3, 8).sum(axis=3)).max() <= 1e-13


def test_bwd_magnitudes_bound_the_gradients_and_head_subset():
    q, k, v = inputs.prefill_inputs(1, 10, 10, 4, 2, 8, torch.float64, seed=14)
    do = _rand(q.shape, 15)
    dq, dk, dv, (mq, mk, mv) = oracle.attention_bwd(q, k, v, do, True, 0.3, with_magnitudes=True)
    assert np.all(mq >= np.abs(dq)) and np.all(mk >= np.abs(dk)) and np.all(mv >= np.abs(dv))
    sq, sk, sv = oracle.attention_bwd(q, k, v, do, True, 0.3, kv_heads=[1])
    assert np.array_equal(sq[:, :, 2:], dq[:, :, 2:]) and np.all(sq[:, :, :2] == 0)
    assert np.array_equal(sk[:, :, 1], dk[:, :, 1]) and np.array_equal(sv[:, :, 1], dv[:, :, 1])


MAG_CASES = [
    # (B, Hq, Hkv, N, Nk, causal)
    (1, 2, 1, 3, 4, False),
    (1, 2, 1, 4, 3, True),       # N > Nk: a leading row sees no key
    (2, 4, 2, 3, 5, True),       # GQA groups of 2, bottom-right causal
]


def _magnitudes_vs_brute(fn, case, seed=7):
    B, Hq, Hkv, N, Nk, causal = case
    d, scale = 4, 0.6
    q, k, v = inputs.prefill_inputs(B, N, Nk, Hq, Hkv, d, torch.float64, seed=seed)
    do = _rand(q.shape, seed + 1)
    _, _, _, (mq, mk, mv) = fn(q, k, v, do, causal, scale, with_magnitudes=True)
    bq, bk, bv = brute.bwd_magnitudes(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, scale)
    worst = 0.0
    for got, ref in ((mq, bq), (mk, bk), (mv, bv)):
        ref = np.asarray(ref)
        worst = max(worst, float(np.abs(got - ref).max() / max(1.0, np.abs(ref).max())))
    return worst


@pytest.mark.parametrize("case", MAG_CASES, ids=lambda c: "B%dHq%dHkv%dN%dNk%d%s" % (c[:5] + ("c" if c[5] else "",)))
def test_bwd_magnitudes_match_the_scalar_brute_force(case):
    """The magnitude sums that set every backward GPU tolerance equal, at
    1e-12, the same sums taken term by term in plain Python loops: pinned from
    above as well as from below."""
    assert _magnitudes_vs_brute(oracle.attention_bwd, case) <= 1e-12


# Planted mistakes in the magnitude sums (each would loosen every backward
# tolerance without failing the gradient pins): the scalar brute force above
# must reject each.
BWD_MUTANTS = {
    "scale dropped from mq": ("mq[b, :, h, :] = scale * ((aS + a * P) @ np.abs(Kg))",
                              "mq[b, :, h, :] = ((aS + a * P) @ np.abs(Kg))"),
    "scale dropped from mk": ("mk[b, :, g, :] += scale * ((aS + a * P).T @ np.abs(Qh))",
                              "mk[b, :, g, :] += ((aS + a * P).T @ np.abs(Qh))"),
    "D term doubled": ("a = np.abs(dOh * (P @ Vg)).sum(axis=1, keepdims=True)",
                       "a = 2 * np.abs(dOh * (P @ Vg)).sum(axis=1, keepdims=True)"),
    "D term dropped": ("mq[b, :, h, :] = scale * ((aS + a * P) @ np.abs(Kg))",
                       "mq[b, :, h, :] = scale * (aS @ np.abs(Kg))"),
    "dV magnitude without abs": ("mv[b, :, g, :] += P.T @ np.abs(dOh)", "mv[b, :, g, :] += P.T @ dOh"),
}


def _mutant_bwd(old, new):
    """attention_bwd from a copy of oracle.py's source with one edit (the copy is
    executed on the CPU in its own namespace; the oracle itself is unchanged)."""
    import os
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.py")).read()
    assert src.count(old) == 1, old
    ns = {"__name__": "oracle_bwd_mutant", "__file__": oracle.__file__}
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), ns)
    return ns["attention_bwd"]


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_magnitude_mutants_are_caught(name):
    fn = _mutant_bwd(*BWD_MUTANTS[name])
    assert max(_magnitudes_vs_brute(fn, c) for c in MAG_CASES) > 1e-6, name


def test_bwd_magnitude_mutant_harness_accepts_the_oracle():
    fn = _mutant_bwd("mv[b, :, g, :] += P.T @ np.abs(dOh)", "mv[b, :, g, :] += P.T @ np.abs(dOh)")
    assert max(_magnitudes_vs_brute(fn, c) for c in MAG_CASES) <= 1e-12

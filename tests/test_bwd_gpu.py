"""Parity of the backward (fa_bwd, through the C ABI) with the fp64 oracle's
chain rule of exact attention.

Tolerance.  bf16 round-to-nearest-even has unit roundoff u = 2^-8.  Each
gradient element is a sum of products in which one factor was rounded to bf16
before its MFMA (P for dV, dS for dK and dQ: relative error <= u each),
accumulated in fp32 (at most n 2^-24 of the sum of the absolute terms, which is
2^-11 of it for n <= 8192 keys or rows) and rounded to bf16 on output (<= u of
the result); dS also carries the error of D = dO.O computed in fp32 from the
bf16-rounded O of the forward (<= u a_i, a_i = sum_d |dO_id O_id|), which
reaches dq and dk as P_ij times that error.  With ``mag`` the oracle's bound of
these terms in absolute value (|dS| and a_i P against |K| or |Q|, P against
|dO|; pinned by a scalar brute force on the CPU), the error of an element is
at most u |ref| + (u + 2^-11) mag, plus the fp32 rounding of the recomputed P
(about 2^-22 relative).  The tests allow u |ref| + 2u mag + 1e-6 and report the
largest err / (|ref| + mag) seen.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import binding, inputs
from oracle import oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -8                     # bf16 unit roundoff
REL_REF, REL_MAG = U, 2 * U


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def gpu_fwd_bwd(q, k, v, do, causal, scale):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = binding.fwd(qd, kd, vd, causal, scale)
    dq, dk, dv = binding.bwd(qd, kd, vd, o, lse, dod, causal, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def assert_grad_close(got, ref, mag, what):
    got = got.double().numpy()
    assert not np.isnan(got).any(), "%s: NaN" % what
    err = np.abs(got - ref)
    bound = np.abs(ref) + mag
    worst = float((err / np.maximum(bound, 1e-30)).max(initial=0.0))
    allowed = REL_REF * np.abs(ref) + REL_MAG * mag + 1e-6
    _say("  %s: max abs err %.3g, max err/(|ref|+mag) %.3g, max err/allowed %.3g, max |ref| %.3g"
         % (what, float(err.max(initial=0.0)), worst, float((err / allowed).max(initial=0.0)),
            float(np.abs(ref).max(initial=0.0))))
    bad = err > allowed
    assert not bad.any(), "%s: %d elements out of tolerance, first at %s" % (
        what, int(bad.sum()), np.unravel_index(np.argmax(bad), bad.shape))


def _dout(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


BWD_SHAPES = [
    # (B, Hq, Hkv, N, Nk)
    (2, 4, 2, 200, 200),
    (1, 8, 1, 77, 530),       # N < Nk: bottom-right causal, a group of 8
    (1, 2, 2, 530, 77),       # N > Nk: leading causal rows see no key
    (1, 4, 4, 1, 1),
    (1, 2, 1, 129, 300),      # tile tails on both sides
    (1, 16, 1, 300, 333),     # a group of 16 heads walked innermost, ragged tiles
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "B%dHq%dHkv%dN%dNk%d" % s)
def test_bwd_shapes(shape, causal, d):
    B, Hq, Hkv, N, Nk = shape
    _say("case: bwd B=%d Hq=%d Hkv=%d N=%d Nk=%d d=%d causal=%s" % (B, Hq, Hkv, N, Nk, d, causal))
    q, k, v = inputs.prefill_inputs(B, N, Nk, Hq, Hkv, d, torch.bfloat16, seed=N + Nk + d + causal)
    do = _dout(q.shape, N + 1)
    scale = inputs.fp32_scale(d)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, causal, scale)
    rq, rk, rv, (mq, mk, mv) = oracle.attention_bwd(q, k, v, do, causal, scale, with_magnitudes=True)
    assert_grad_close(dq, rq, mq, "dQ")
    assert_grad_close(dk, rk, mk, "dK")
    assert_grad_close(dv, rv, mv, "dV")


def test_bwd_rows_without_keys_and_masked_keys_bitwise():
    """Causal, N > Nk: rows that see no key get dq = 0 exactly, and replacing
    every masked (future) key's K and V by other finite values changes no
    gradient of the visible ones, bit for bit (dk, dv of those keys aside)."""
    q, k, v = inputs.prefill_inputs(1, 300, 200, 4, 2, 128, torch.bfloat16, seed=31)
    do = _dout(q.shape, 32)
    scale = inputs.fp32_scale(128)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, True, scale)
    assert torch.all(dq[:, :100] == 0)
    # query rows 100..149 (offset -100) see keys up to 49: perturb keys >= 50
    # and compare the gradients that cannot depend on them
    k2, v2 = k.clone(), v.clone()
    g = torch.Generator().manual_seed(33)
    k2[:, 50:] = torch.randn(k2[:, 50:].shape, generator=g).to(torch.bfloat16)
    v2[:, 50:] = torch.randn(v2[:, 50:].shape, generator=g).to(torch.bfloat16)
    dq2, dk2, dv2 = gpu_fwd_bwd(q, k2, v2, do, True, scale)
    assert torch.equal(dq[:, :150], dq2[:, :150])


def test_bwd_is_deterministic():
    q, k, v = inputs.prefill_inputs(1, 700, 700, 8, 2, 128, torch.bfloat16, seed=34)
    do = _dout(q.shape, 35)
    a = gpu_fwd_bwd(q, k, v, do, True, 0.1)
    b = gpu_fwd_bwd(q, k, v, do, True, 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_llama70b_shape_one_kv_head_full_size():
    """The C4 workload shape (B1 Hq64 Hkv8 N=Nk=8192 d128, causal): the
    gradients of kv head 0 (dk, dv, and dq of its 8 query heads) against the
    oracle, and the rest finite."""
    cfg = inputs.LLAMA70B_GQA_BF16
    _say("case: bwd %s (kv head 0 checked)" % cfg.name)
    q, k, v = inputs.prefill_config_inputs(cfg)
    do = _dout(q.shape, 36)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, cfg.causal, cfg.scale)
    G = cfg.Hq // cfg.Hkv
    rq, rk, rv, (mq, mk, mv) = oracle.attention_bwd(q[:, :, :G], k[:, :, :1], v[:, :, :1], do[:, :, :G],
                                                    cfg.causal, cfg.scale, with_magnitudes=True)
    assert_grad_close(dq[:, :, :G], rq, mq, "dQ (heads 0-7)")
    assert_grad_close(dk[:, :, :1], rk, mk, "dK (kv head 0)")
    assert_grad_close(dv[:, :, :1], rv, mv, "dV (kv head 0)")
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_no_queries_gives_zero_key_gradients(causal):
    """N = 0 with keys present: no query sees any key, so dk = dv = 0; the
    outputs start as NaN so that an unwritten element shows."""
    d = 128
    q = torch.zeros((1, 0, 4, d), dtype=torch.bfloat16, device="cuda")
    k = _dout((1, 64, 2, d), 40).cuda()
    v = _dout((1, 64, 2, d), 41).cuda()
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 4, 0), dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    binding.bwd(q, k, v, o, lse, o, causal, inputs.fp32_scale(d), dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)

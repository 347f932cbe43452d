"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Tolerances (max abs error against the fp64 oracle): fp32 inputs 1e-5 on O and
LSE; bf16 inputs 1e-2 on O and 1e-3 on LSE.  LSE = -inf on both sides counts as
equal; any NaN fails.  Masking and cache indexing are checked bit for bit.
"""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import binding, inputs
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (1e-2, 1e-3)}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.load_library()          # raises if libfa.so is missing: no fallback path
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def gpu_fwd(q, k, v, causal, scale):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = binding.fwd(qd, kd, vd, causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_decode(q, kc, vc, cu, max_len, scale):
    o, lse = binding.decode(q.cuda(), kc.cuda(), vc.cuda(), cu.cuda(), max_len, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def assert_close(got, ref, tol, what, rel=0.0):
    """max |got - ref| <= tol + rel*|ref| elementwise (rel = 0 for the stated tolerances)."""
    got = np.asarray(got.double() if torch.is_tensor(got) else got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert not np.isnan(got).any(), "%s: NaN in GPU output" % what
    same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(got - ref) - rel * np.abs(ref))
    worst = float(err.max(initial=0.0))
    _say("  %s: max abs err %.3g (tol %.1g)" % (what, worst, tol))
    assert worst <= tol, "%s: max abs err %g > %g at %s" % (what, worst, tol,
                                                             np.unravel_index(err.argmax(), err.shape))


def check_full(q, k, v, causal, scale):
    o, lse = gpu_fwd(q, k, v, causal, scale)
    ro, rlse = oracle.attention(q, k, v, causal, scale)
    tol_o, tol_l = TOL[q.dtype]
    assert_close(o, ro, tol_o, "O")
    assert_close(lse, rlse, tol_l, "LSE")
    return o, lse


# ------------------------------------------------------------------ workloads

def test_workload_single_head_fp32():
    cfg = inputs.SINGLE_HEAD_F32
    _say("case: %s" % cfg.name)
    check_full(*inputs.prefill_config_inputs(cfg), cfg.causal, cfg.scale)


def test_workload_bert_large_bf16():
    cfg = inputs.BERT_LARGE_BF16
    _say("case: %s" % cfg.name)
    check_full(*inputs.prefill_config_inputs(cfg), cfg.causal, cfg.scale)


def test_workload_gpt2_causal_bf16():
    cfg = inputs.GPT2_CAUSAL_BF16
    _say("case: %s" % cfg.name)
    check_full(*inputs.prefill_config_inputs(cfg), cfg.causal, cfg.scale)


def _c4_rows(cfg, rng):
    heads = [0, 1, 7, 8, 31, 56, 63]
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, 257, 1023, 4095, 4096, 8127, 8128, 8190, 8191]
    rows = [(0, h, i) for h in heads for i in fixed]
    rows += [(0, int(rng.integers(cfg.Hq)), int(rng.integers(cfg.N))) for _ in range(64)]
    return np.array(rows)


def test_workload_llama70b_gqa_full_size():
    """Full-size launch (the one the benchmark times).  Every element of kv
    group 0 (query heads 0-7, all 8192 rows: a whole GQA group, one XCD's share
    of the work order) against the oracle; sampled rows of the other heads; and
    properties that hold on every row."""
    cfg = inputs.LLAMA70B_GQA_BF16
    _say("case: %s (kv group 0 in full, other heads sampled)" % cfg.name)
    q, k, v = inputs.prefill_config_inputs(cfg)
    o, lse = gpu_fwd(q, k, v, cfg.causal, cfg.scale)
    G = cfg.Hq // cfg.Hkv
    ro, rl = oracle.attention(q[:, :, :G].contiguous(), k[:, :, :1].contiguous(), v[:, :, :1].contiguous(),
                              cfg.causal, cfg.scale)
    assert_close(o[:, :, :G], ro, 1e-2, "O (heads 0-7, every row)")
    assert_close(lse[:, :G], rl, 1e-3, "LSE (heads 0-7, every row)")
    rows = _c4_rows(cfg, np.random.default_rng(0))
    ro, rl = oracle.attention_rows(q, k, v, cfg.causal, cfg.scale, rows)
    got_o = o[rows[:, 0], rows[:, 2], rows[:, 1]]
    got_l = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_close(got_o, ro, 1e-2, "O (sampled rows)")
    assert_close(got_l, rl, 1e-3, "LSE (sampled rows)")
    # every row: finite, O inside the per-column range of V (a convex combination)
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    G = cfg.Hq // cfg.Hkv
    vmin = v.float().amin(dim=1).repeat_interleave(G, dim=1)     # [B, Hq, d]
    vmax = v.float().amax(dim=1).repeat_interleave(G, dim=1)
    of = o.float()
    assert (of >= vmin[:, None] - 1e-2).all() and (of <= vmax[:, None] + 1e-2).all()
    # causal row 0 sees only key 0: O = V[0] bit for bit, in every head
    assert torch.equal(o[:, 0], v[:, 0].repeat_interleave(G, dim=1))


def test_workload_decode_full_size():
    """The decode workload the benchmark times (32 sequences, 492,798 cached
    rows): every element of O and LSE against the oracle."""
    cfg = inputs.DECODE_VARLEN_BF16
    _say("case: %s (every row)" % cfg.name)
    q, kc, vc, cu, lens = inputs.decode_config_inputs(cfg)
    o, lse = gpu_decode(q, kc, vc, cu, int(lens.max()), cfg.scale)
    ro, rl = oracle.decode(q, kc, vc, cu, cfg.scale)
    assert_close(o, ro, 1e-2, "O")
    assert_close(lse, rl, 1e-3, "LSE")


# ------------------------------------------------------------- shape sweep

SHAPES = [
    # (B, Hq, Hkv, N, Nk)
    (2, 4, 2, 300, 300),        # several tiles and a ragged tail
    (1, 8, 1, 77, 530),         # N < Nk: bottom-right causal, group of 8
    (1, 2, 2, 530, 77),         # N > Nk: leading causal rows see no key
    (3, 2, 1, 1, 1),
    (1, 1, 1, 1, 700),
    (2, 16, 16, 257, 257),
    (1, 4, 4, 513, 64),
    (1, 2, 1, 64, 64),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dHq%dHkv%dN%dNk%d" % s)
def test_prefill_shapes(shape, causal, d, dtype):
    B, Hq, Hkv, N, Nk = shape
    _say("case: prefill %s causal=%s d=%d %s" % (shape, causal, d, dtype))
    q, k, v = inputs.prefill_inputs(B, N, Nk, Hq, Hkv, d, dtype, seed=N + Nk + d)
    check_full(q, k, v, causal, inputs.fp32_scale(d))


@pytest.mark.parametrize("N", [4096, 4100], ids=["N4096", "N4100"])
def test_prefill_d64_causal_both_tile_heights(N):
    """Head dim 64, causal: up to N = 4096 the launch uses 128-row workgroups
    (16 rows per wave), above it 384-row ones (48 per wave); both sides of the
    switch against the oracle, with ragged tails for both tile heights."""
    _say("case: prefill d64 causal N=%d" % N)
    q, k, v = inputs.prefill_inputs(1, N, N, 2, 1, 64, torch.bfloat16, seed=N)
    check_full(q, k, v, True, inputs.fp32_scale(64))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_prefill_f32_many_key_tiles_per_wave(causal, d):
    """fp32 splits a workgroup's 32-key tiles over its 8 waves (wave w takes
    tiles w, w+8, ...) and merges their partial softmaxes.  4100 keys (129
    tiles, the last holding 4 keys) give each wave 16 or 17 tiles; 300
    queries against them under the bottom-right causal mask see 3801 to 4100
    keys each, so the mask cuts into the last tiles row by row."""
    _say("case: prefill f32 N=300 Nk=4100 causal=%s d=%d" % (causal, d))
    q, k, v = inputs.prefill_inputs(1, 300, 4100, 4, 2, d, torch.float32, seed=4400 + d)
    check_full(q, k, v, causal, inputs.fp32_scale(d))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_peaked_softmax_rows(dtype):
    """Q scaled by 10: scores spread over about +-30, the running max moves
    often and most weights underflow.  Rows are then dominated by one key, so
    |O| reaches the size of single V entries (up to ~5); rounding O to bf16
    alone costs up to 2^-8 |O| there, which the bf16 bound adds to 1e-2.  In
    fp32 the rounding error of a logit grows with its size, so ten times larger
    logits get ten times the 1e-5 bound."""
    _say("case: peaked softmax %s" % dtype)
    q, k, v = inputs.prefill_inputs(2, 333, 333, 4, 2, 128, dtype, seed=7, q_mult=10.0)
    tol_o, tol_l = TOL[dtype]
    if dtype == torch.float32:
        tol_o, tol_l = 10 * tol_o, 10 * tol_l
    rel = 2.0 ** -8 if dtype == torch.bfloat16 else 0.0
    for causal in (False, True):
        o, lse = gpu_fwd(q, k, v, causal, inputs.fp32_scale(128))
        ro, rl = oracle.attention(q, k, v, causal, inputs.fp32_scale(128))
        assert_close(o, ro, tol_o, "O", rel=rel)
        assert_close(lse, rl, tol_l, "LSE")


@pytest.mark.parametrize("d,B,Hq,Hkv,N", [(64, 1, 4, 2, 700), (128, 1, 4, 2, 700), (64, 1, 2, 1, 4200),
                                           (128, 2, 64, 8, 700)],
                         ids=["d64", "d128", "d64-long", "d128-many-heads"])
def test_scores_jump_past_the_reference(d, B, Hq, Hkv, N):
    """Key magnitudes ramp up along the sequence (x1 at key 0 to x40 at the
    last key, Q x3), so scores of later tiles exceed the reference that tile 0
    set by far more than the lazy-rescale slack, again and again: the
    reference moves and O, l are rescaled many times per row, on unmasked and
    (causal) diagonal tiles alike.  Rows end dominated by one or two keys,
    where the bf16 rounding of the weights (relative error up to u = 2^-8
    each, before the P.V product) no longer averages out: |dO| <= u sum_j
    p_j |V_j| <= u max|V|, and O's own rounding adds u |O|.  So O takes
    u max|V| + u |O|; LSE (up to several hundred) the 1e-3 bound.  The shapes
    cover each workgroup size the launch picks: 128 and 256 rows (the small
    ones), 384 rows at head dim 64 (causal past 4096 rows) and at head dim 128
    (256 or more 384-row tiles)."""
    q, k, v = inputs.prefill_inputs(B, N, N, Hq, Hkv, d, torch.bfloat16, seed=11, q_mult=3.0)
    ramp = torch.linspace(1.0, 40.0, N, dtype=torch.float64).view(1, N, 1, 1)
    k = (k.double() * ramp).to(torch.bfloat16)
    scale = inputs.fp32_scale(d)
    _say("case: scores jump past the reference d=%d B=%d Hq=%d N=%d" % (d, B, Hq, N))
    for causal in (False, True):
        o, lse = gpu_fwd(q, k, v, causal, scale)
        ro, rl = oracle.attention(q, k, v, causal, scale)
        assert float(rl.max()) > 200.0        # the scores did climb far past tile 0's
        assert_close(o, ro, 2.0 ** -8 * float(v.double().abs().max()), "O", rel=2.0 ** -8)
        assert_close(lse, rl, TOL[torch.bfloat16][1], "LSE")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_no_keys_gives_zero_and_minus_inf(dtype):
    q, k, v = inputs.prefill_inputs(2, 5, 0, 2, 1, 64, dtype)
    o, lse = gpu_fwd(q, k, v, False, 0.125)
    assert torch.equal(o, torch.zeros_like(o)) and bool((lse == -math.inf).all())


def test_empty_batch_and_rows_are_noops():
    for B, N in ((0, 16), (2, 0)):
        q, k, v = inputs.prefill_inputs(B, N, 16, 2, 1, 64, torch.bfloat16)
        o, lse = gpu_fwd(q, k, v, True, 0.125)
        assert o.numel() == 0 and lse.numel() == 0


# ----------------------------------------------------------- bitwise pins

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_masked_keys_have_no_effect_bitwise(dtype, d):
    """Causal: rows <= r never see keys > r, so replacing those K/V rows with
    other finite values leaves rows <= r unchanged bit for bit."""
    B, Hq, Hkv, N = 1, 4, 2, 300
    q, k, v = inputs.prefill_inputs(B, N, N, Hq, Hkv, d, dtype, seed=3)
    o1, l1 = gpu_fwd(q, k, v, True, inputs.fp32_scale(d))
    r = 137
    k2, v2 = k.clone(), v.clone()
    g = torch.Generator().manual_seed(99)
    k2[:, r + 1:] = (torch.randn(k2[:, r + 1:].shape, generator=g) * 3).to(dtype)
    v2[:, r + 1:] = (torch.randn(v2[:, r + 1:].shape, generator=g) * 3).to(dtype)
    o2, l2 = gpu_fwd(q, k2, v2, True, inputs.fp32_scale(d))
    assert torch.equal(o1[:, :r + 1], o2[:, :r + 1])
    assert torch.equal(l1[:, :, :r + 1], l2[:, :, :r + 1])
    assert not torch.equal(o1[:, r + 1:], o2[:, r + 1:])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("d", [64, 128])
def test_rows_past_the_end_are_never_read(d, causal, dtype):
    """K and V are the first Nk rows of a larger allocation whose remaining
    rows hold NaN (Nk is not a multiple of any tile size, so the last tile is
    ragged).  A kernel that read any row past Nk, even only to multiply it by a
    zero weight, would put NaN into O; the output must match the oracle."""
    B, Hq, Hkv, N, Nk = 1, 4, 2, 150, 333
    q, k, v = inputs.prefill_inputs(B, N, Nk, Hq, Hkv, d, dtype, seed=21)
    pad = 200
    kbig = torch.full((B, Nk + pad, Hkv, d), float("nan"), dtype=dtype, device="cuda")
    vbig = torch.full((B, Nk + pad, Hkv, d), float("nan"), dtype=dtype, device="cuda")
    kbig[:, :Nk] = k.cuda()
    vbig[:, :Nk] = v.cuda()
    kd, vd = kbig[:, :Nk], vbig[:, :Nk]
    assert kd.is_contiguous() and vd.is_contiguous()
    o, lse = binding.fwd(q.cuda(), kd, vd, causal, inputs.fp32_scale(d))
    torch.cuda.synchronize()
    ro, rlse = oracle.attention(q, k, v, causal, inputs.fp32_scale(d))
    tol_o, tol_l = TOL[dtype]
    assert_close(o.cpu(), ro, tol_o, "O")
    assert_close(lse.cpu(), rlse, tol_l, "LSE")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_first_causal_row_returns_v0_bitwise(dtype):
    q, k, v = inputs.prefill_inputs(2, 129, 129, 8, 2, 128, dtype, seed=4)
    o, lse = gpu_fwd(q, k, v, True, inputs.fp32_scale(128))
    assert torch.equal(o[:, 0], v[:, 0].repeat_interleave(4, dim=1))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_visible_key_count_is_exact(dtype):
    """Q = 0: every visible score is 0, so LSE_i = ln(#visible keys); an
    off-by-one in the mask moves LSE by at least 1/Nk."""
    for N, Nk in ((300, 300), (100, 333)):
        q = torch.zeros(1, N, 2, 64, dtype=dtype)
        _, k, v = inputs.prefill_inputs(1, N, Nk, 2, 2, 64, dtype, seed=5)
        _, lse = gpu_fwd(q, k, v, True, 0.125)
        expect = torch.log(torch.arange(1, N + 1, dtype=torch.float64) + (Nk - N))
        assert (lse.double() - expect).abs().max() <= 1e-5
        _, lse = gpu_fwd(q, k, v, False, 0.125)
        assert (lse.double() - math.log(Nk)).abs().max() <= 1e-5


def test_gqa_equals_repeated_kv_heads_bitwise():
    q, k, v = inputs.prefill_inputs(1, 200, 200, 16, 2, 128, torch.bfloat16, seed=6)
    for causal in (False, True):
        o1, l1 = gpu_fwd(q, k, v, causal, inputs.fp32_scale(128))
        o2, l2 = gpu_fwd(q, k.repeat_interleave(8, dim=2).contiguous(),
                         v.repeat_interleave(8, dim=2).contiguous(), causal, inputs.fp32_scale(128))
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeated_runs_are_bitwise_identical():
    q, k, v = inputs.prefill_inputs(1, 1000, 1000, 8, 1, 128, torch.bfloat16, seed=8)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref = binding.fwd(qd, kd, vd, True, inputs.fp32_scale(128))
    for _ in range(5):
        o, lse = binding.fwd(qd, kd, vd, True, inputs.fp32_scale(128))
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])


# ----------------------------------------------------------------- decode

DECODE_CASES = [
    # (lens, Hq, Hkv, d)
    ([1, 7, 64, 65, 255, 256, 257, 1000, 3000, 0, 5000], 64, 8, 128),
    ([1, 7, 64, 65, 255, 256, 257, 1000, 3000, 0, 5000], 32, 4, 64),
    ([300, 1, 2049], 16, 1, 128),
    ([33, 4100], 4, 4, 128),
    ([0, 0, 0], 8, 8, 64),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "Hq%dHkv%dd%d" % c[1:])
def test_decode_shapes(case):
    lens, Hq, Hkv, d = case
    _say("case: decode lens=%s Hq=%d Hkv=%d d=%d" % case)
    q, kc, vc, cu = inputs.decode_inputs(lens, Hq, Hkv, d, torch.bfloat16, seed=len(lens) + d)
    for max_len in (max(lens), max(lens) + 777):
        o, lse = gpu_decode(q, kc, vc, cu, max_len, inputs.fp32_scale(d))
        ro, rl = oracle.decode(q, kc, vc, cu, inputs.fp32_scale(d))
        assert_close(o, ro, 1e-2, "O")
        assert_close(lse, rl, 1e-3, "LSE")


def test_decode_other_sequences_have_no_effect_bitwise():
    lens = [900, 1500, 700]
    q, kc, vc, cu = inputs.decode_inputs(lens, 64, 8, 128, torch.bfloat16, seed=10)
    o1, l1 = gpu_decode(q, kc, vc, cu, 1500, inputs.fp32_scale(128))
    kc2, vc2 = kc.clone(), vc.clone()
    g = torch.Generator().manual_seed(1)
    s, e = int(cu[1]), int(cu[2])
    kc2[s:e] = (torch.randn(kc2[s:e].shape, generator=g) * 2).to(torch.bfloat16)
    vc2[s:e] = (torch.randn(vc2[s:e].shape, generator=g) * 2).to(torch.bfloat16)
    o2, l2 = gpu_decode(q, kc2, vc2, cu, 1500, inputs.fp32_scale(128))
    for b in (0, 2):
        assert torch.equal(o1[b], o2[b]) and torch.equal(l1[b], l2[b])
    assert not torch.equal(o1[1], o2[1])


def test_decode_cache_rows_past_the_end_are_never_read():
    """The packed caches are the first sum(L) rows of larger allocations whose
    remaining rows hold NaN; reading any of them would put NaN into O."""
    lens = [37, 1000, 2049, 333]
    Hq, Hkv, d = 16, 2, 128
    q, kc, vc, cu = inputs.decode_inputs(lens, Hq, Hkv, d, torch.bfloat16, seed=13)
    total, pad = int(cu[-1]), 300
    kbig = torch.full((total + pad, Hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vbig = torch.full((total + pad, Hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    kbig[:total] = kc.cuda()
    vbig[:total] = vc.cuda()
    o, lse = binding.decode(q.cuda(), kbig[:total], vbig[:total], cu.cuda(), max(lens), inputs.fp32_scale(d))
    torch.cuda.synchronize()
    ro, rl = oracle.decode(q, kc, vc, cu, inputs.fp32_scale(d))
    assert_close(o.cpu(), ro, 1e-2, "O")
    assert_close(lse.cpu(), rl, 1e-3, "LSE")


def test_decode_visible_count_is_exact():
    lens = [1, 513, 2048, 7777]
    q, kc, vc, cu = inputs.decode_inputs(lens, 16, 2, 128, torch.bfloat16, seed=11)
    q.zero_()
    _, lse = gpu_decode(q, kc, vc, cu, 7777, 0.1)
    expect = torch.log(torch.tensor(lens, dtype=torch.float64))[:, None]
    assert (lse.double() - expect).abs().max() <= 1e-5


def test_decode_matches_single_query_prefill():
    lens = [700, 1300]
    q, kc, vc, cu = inputs.decode_inputs(lens, 16, 2, 128, torch.bfloat16, seed=12)
    o, lse = gpu_decode(q, kc, vc, cu, 1300, inputs.fp32_scale(128))
    for b, L in enumerate(lens):
        s = int(cu[b])
        op, lp = gpu_fwd(q[b:b + 1, None].contiguous(), kc[None, s:s + L].contiguous(),
                         vc[None, s:s + L].contiguous(), False, inputs.fp32_scale(128))
        assert (o[b].float() - op[0, 0].float()).abs().max() <= 1e-2
        assert (lse[b] - lp[0, :, 0]).abs().max() <= 1e-3



@pytest.mark.parametrize("fill", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_decode_fewer_keys_than_ranges_with_dirty_workspace(fill):
    """When the cache holds fewer keys than the plan has key ranges (short
    caches with a large max_seqlen_k bound), some ranges are empty; the merge
    must not read a partial slot that no range wrote.  The workspace starts
    filled with NaN or Inf, as reused memory may be."""
    lens = [1000] + [1] * 63
    Hq, Hkv, d = 8, 1, 128
    _say("case: decode, fewer keys than ranges, workspace filled with %s" % fill)
    q, kc, vc, cu = inputs.decode_inputs(lens, Hq, Hkv, d, torch.bfloat16, seed=31)
    total, rows = int(cu[-1]), 8192
    kbig = torch.zeros((rows, Hkv, d), dtype=torch.bfloat16, device="cuda")
    vbig = torch.zeros((rows, Hkv, d), dtype=torch.bfloat16, device="cuda")
    kbig[:total] = kc.cuda()
    vbig[:total] = vc.cuda()
    max_len = rows                                        # a valid upper bound of every length
    ws_bytes = binding.decode_workspace_bytes(len(lens), Hq, Hkv, d, max_len)
    ws = torch.full(((ws_bytes + 3) // 4,), fill, dtype=torch.float32, device="cuda").view(torch.uint8)
    o, lse = binding.decode(q.cuda(), kbig, vbig, cu.cuda(), max_len, inputs.fp32_scale(d), workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(q, kc, vc, cu, inputs.fp32_scale(d))
    assert_close(o.cpu(), ro, 1e-2, "O")
    assert_close(lse.cpu(), rl, 1e-3, "LSE")


# --------------------------------------------- paged cache, new row appended

def gpu_decode_paged(x, scale, append=True, table=None):
    """Runs fa_decode_paged on the dict of ``inputs.paged_decode_inputs``;
    returns (o, lse, k_pages after, v_pages after) on the CPU."""
    kp, vp = x["k_pages"].cuda(), x["v_pages"].cuda()
    tbl = (x["block_table"] if table is None else table).cuda()
    kn = x["k_new"].cuda() if append else None
    vn = x["v_new"].cuda() if append else None
    max_len = int(x["seqlens"].max()) if x["seqlens"].numel() else 0
    o, lse = binding.decode_paged(x["q"].cuda(), kp, vp, tbl, x["seqlens"].cuda(), max_len, scale, kn, vn)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), kp.cpu(), vp.cpu()


def _bits(t):
    return t.view(torch.int16)


def expected_pages(x, append=True):
    """The pages after the call: unchanged, plus (appending) each sequence's new
    row at logical row L_b of its table (layout only, no arithmetic)."""
    kp, vp = x["k_pages"].clone(), x["v_pages"].clone()
    if append:
        bs = kp.shape[1]
        for b, L in enumerate(x["seqlens"].tolist()):
            pb = int(x["block_table"][b, L // bs])
            kp[pb, L % bs] = x["k_new"][b]
            vp[pb, L % bs] = x["v_new"][b]
    return kp, vp


PAGED_CASES = [
    # (lens, Hq, Hkv, d, block_size): empty caches, one row, tile and block edges
    ([0, 1, 31, 32, 33, 63, 64, 65, 1000, 0], 64, 8, 128, 32),
    ([0, 1, 31, 32, 33, 63, 64, 65, 1000, 3000], 32, 4, 64, 64),
    ([255, 256, 257, 2049], 16, 2, 128, 256),
    ([5, 4100], 4, 4, 128, 1024),
]


@pytest.mark.parametrize("append", [True, False], ids=["append", "no_append"])
@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: "Hq%dHkv%dd%dbs%d" % c[1:])
def test_paged_decode(case, append):
    """O and LSE against the oracle over the L_b (+1 appended) rows; the pages
    afterwards hold exactly the expected rows, bit for bit, including the NaN
    fill of unused rows (none of which may be read)."""
    lens, Hq, Hkv, d, bs = case
    _say("case: paged decode lens=%s Hq=%d Hkv=%d d=%d block_size=%d append=%s" % (lens, Hq, Hkv, d, bs, append))
    x = inputs.paged_decode_inputs(lens, Hq, Hkv, d, bs, torch.bfloat16, seed=sum(lens) % 97 + d)
    scale = inputs.fp32_scale(d)
    o, lse, kp, vp = gpu_decode_paged(x, scale, append)
    if append:
        ro, rl, _, _, _ = oracle.decode_append(x["q"], x["kc"], x["vc"], x["cu"], x["k_new"], x["v_new"], scale)
    else:
        ro, rl = oracle.decode(x["q"], x["kc"], x["vc"], x["cu"], scale)
    assert_close(o, ro, 1e-2, "O")
    assert_close(lse, rl, 1e-3, "LSE")
    ek, ev = expected_pages(x, append)
    assert torch.equal(_bits(kp), _bits(ek)) and torch.equal(_bits(vp), _bits(ev))


def test_paged_decode_other_sequences_have_no_effect_bitwise():
    lens = [900, 1500, 700]
    x = inputs.paged_decode_inputs(lens, 64, 8, 128, 64, torch.bfloat16, seed=21)
    o1, l1, _, _ = gpu_decode_paged(x, inputs.fp32_scale(128))
    y = dict(x)
    y["k_pages"], y["v_pages"] = x["k_pages"].clone(), x["v_pages"].clone()
    g = torch.Generator().manual_seed(2)
    for pb in x["block_table"][1].tolist():
        if pb >= 0:
            y["k_pages"][pb] = (torch.randn(y["k_pages"][pb].shape, generator=g) * 2).to(torch.bfloat16)
            y["v_pages"][pb] = (torch.randn(y["v_pages"][pb].shape, generator=g) * 2).to(torch.bfloat16)
    o2, l2, _, _ = gpu_decode_paged(y, inputs.fp32_scale(128))
    for b in (0, 2):
        assert torch.equal(o1[b], o2[b]) and torch.equal(l1[b], l2[b])
    assert not torch.equal(o1[1], o2[1])


def test_paged_decode_entry_outside_the_cache_is_an_absent_block():
    """A block-table entry outside [0, num_blocks) breaks the precondition; its
    block is then neither read nor written and its rows count as absent keys."""
    lens = [200, 300]
    bs = 64
    x = inputs.paged_decode_inputs(lens, 16, 2, 128, bs, torch.bfloat16, seed=22)
    table = x["block_table"].clone()
    nb = x["k_pages"].shape[0]
    table[1, 1] = nb + 5                                  # rows 64..127 of sequence 1
    o, lse, kp, vp = gpu_decode_paged(x, inputs.fp32_scale(128), table=table)
    keep = [i for i in range(lens[1]) if not bs <= i < 2 * bs]
    s1 = int(x["cu"][1])
    kc = torch.cat([x["kc"][:s1], x["kc"][s1:][keep]])
    vc = torch.cat([x["vc"][:s1], x["vc"][s1:][keep]])
    cu = inputs.cu_from_lengths([lens[0], len(keep)])
    ro, rl, _, _, _ = oracle.decode_append(x["q"], kc, vc, cu, x["k_new"], x["v_new"], inputs.fp32_scale(128))
    assert_close(o, ro, 1e-2, "O")
    assert_close(lse, rl, 1e-3, "LSE")
    ek, ev = expected_pages(x, True)
    assert torch.equal(_bits(kp), _bits(ek)) and torch.equal(_bits(vp), _bits(ev))


@pytest.mark.parametrize("fill", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_paged_decode_fewer_tiles_than_ranges_with_dirty_workspace(fill):
    """One long and many one-row caches on one kv head: the plan has more key
    ranges (2048) than the cache has 32-key tiles, so some ranges are empty and
    the merge must skip them without reading an unwritten partial slot.  The
    workspace starts filled with NaN or Inf."""
    lens = [32768 - 1] + [32] * 63
    Hq, Hkv, d, bs = 8, 1, 128, 64
    _say("case: paged decode, fewer tiles than ranges, workspace filled with %s" % fill)
    x = inputs.paged_decode_inputs(lens, Hq, Hkv, d, bs, torch.bfloat16, seed=32)
    scale = inputs.fp32_scale(d)
    max_len = max(lens)
    B = len(lens)
    ws_bytes = binding.decode_paged_workspace_bytes(B, Hq, Hkv, d, max_len)
    ws = torch.full(((ws_bytes + 3) // 4,), fill, dtype=torch.float32, device="cuda").view(torch.uint8)
    kp, vp = x["k_pages"].cuda(), x["v_pages"].cuda()
    o, lse = binding.decode_paged(x["q"].cuda(), kp, vp, x["block_table"].cuda(), x["seqlens"].cuda(), max_len,
                                  scale, x["k_new"].cuda(), x["v_new"].cuda(), workspace=ws)
    torch.cuda.synchronize()
    ro, rl, _, _, _ = oracle.decode_append(x["q"], x["kc"], x["vc"], x["cu"], x["k_new"], x["v_new"], scale)
    assert_close(o.cpu(), ro, 1e-2, "O")
    assert_close(lse.cpu(), rl, 1e-3, "LSE")


def test_paged_decode_workload_full_size():
    """The decode workload's lengths, Q, K and V on a paged cache of 64-row
    blocks, one new row appended per sequence: every element of O and LSE
    against the oracle, and every page row checked after the append."""
    cfg = inputs.DECODE_VARLEN_BF16
    _say("case: %s, paged (64-row blocks), new row appended (every row)" % cfg.name)
    x = inputs.paged_config_inputs(cfg, 64, fill=float("nan"))
    o, lse, kp, vp = gpu_decode_paged(x, cfg.scale)
    ro, rl, _, _, _ = oracle.decode_append(x["q"], x["kc"], x["vc"], x["cu"], x["k_new"], x["v_new"], cfg.scale)
    assert_close(o, ro, 1e-2, "O")
    assert_close(lse, rl, 1e-3, "LSE")
    ek, ev = expected_pages(x, True)
    assert torch.equal(_bits(kp), _bits(ek)) and torch.equal(_bits(vp), _bits(ev))


# ------------------------------------------------- variable-length / chunked prefill

def gpu_fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, causal, scale):
    o, lse = binding.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max_q, max_k,
                                causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


VARLEN_CASES = [
    # (q_lens, k_lens, Hq, Hkv): a single row; a chunk on a longer cache; an
    # empty chunk; a square ragged sequence; a chunk with no keys; a short chunk
    # on a long cache; more queries than keys (causal: the leading rows see none)
    ((1, 37, 0, 401, 200, 64, 530), (1, 300, 50, 401, 0, 1000, 77), 8, 2),
    # query-tile boundaries (384 rows per workgroup) and key-tile tails
    ((384, 385, 767), (384, 1000, 767), 4, 4),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", VARLEN_CASES, ids=["mixed", "tile_edges"])
def test_varlen_prefill(case, causal, d):
    q_lens, k_lens, Hq, Hkv = case
    _say("case: varlen q_lens=%s k_lens=%s Hq=%d Hkv=%d d=%d causal=%s" % (q_lens, k_lens, Hq, Hkv, d, causal))
    q, k, v, cu_q, cu_k = inputs.varlen_inputs(q_lens, k_lens, Hq, Hkv, d, torch.bfloat16, seed=d + causal)
    scale = inputs.fp32_scale(d)
    o, lse = gpu_fwd_varlen(q, k, v, cu_q, cu_k, max(q_lens), max(k_lens), causal, scale)
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale)
    assert_close(o, ro, 1e-2, "O")
    assert_close(lse, rl, 1e-3, "LSE")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_equal_lengths_match_fixed_length_bitwise(causal):
    """Packed equal-length sequences give the fixed-length launch's results bit for bit."""
    B, N, Nk, Hq, Hkv, d = 3, 500, 700, 8, 2, 128
    q, k, v = inputs.prefill_inputs(B, N, Nk, Hq, Hkv, d, torch.bfloat16, seed=5)
    scale = inputs.fp32_scale(d)
    o, lse = gpu_fwd(q, k, v, causal, scale)
    vo, vl = gpu_fwd_varlen(q.reshape(B * N, Hq, d), k.reshape(B * Nk, Hkv, d), v.reshape(B * Nk, Hkv, d),
                            inputs.cu_from_lengths([N] * B), inputs.cu_from_lengths([Nk] * B), N, Nk, causal, scale)
    assert torch.equal(vo, o.reshape(B * N, Hq, d))
    assert torch.equal(vl, lse.transpose(0, 1).reshape(Hq, B * N))


def test_varlen_other_sequences_have_no_effect_bitwise():
    """NaN in every row of the other sequences leaves a sequence's result unchanged
    bit for bit: its workgroups read only its own rows."""
    q_lens, k_lens = (300, 129, 512), (900, 129, 700)
    q, k, v, cu_q, cu_k = inputs.varlen_inputs(q_lens, k_lens, 8, 2, 128, torch.bfloat16, seed=9)
    scale = inputs.fp32_scale(128)
    o, lse = gpu_fwd_varlen(q, k, v, cu_q, cu_k, 512, 900, True, scale)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:300] = float("nan")
    q2[429:] = float("nan")
    k2[:900] = float("nan")
    k2[1029:] = float("nan")
    v2[:900] = float("nan")
    v2[1029:] = float("nan")
    o2, lse2 = gpu_fwd_varlen(q2, k2, v2, cu_q, cu_k, 512, 900, True, scale)
    assert torch.equal(o[300:429], o2[300:429])
    assert torch.equal(lse[:, 300:429], lse2[:, 300:429])


def test_varlen_chunked_workload_full_size():
    """The chunked-prefill workload the benchmark times, at full size; the oracle
    checks sampled rows (first, last and random rows of every sequence) one by
    one, and every element of the sequence with the shortest cached prefix."""
    cfg = inputs.VARLEN_CHUNKED_BF16
    _say("case: %s (sampled rows)" % cfg.name)
    q, k, v, cu_q, cu_k, q_lens, k_lens = inputs.varlen_config_inputs(cfg)
    o, lse = gpu_fwd_varlen(q, k, v, cu_q, cu_k, int(q_lens.max()), int(k_lens.max()), cfg.causal, cfg.scale)
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    rng = np.random.default_rng(1)
    cq, ck = cu_q.tolist(), cu_k.tolist()
    for b in range(cfg.B):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        n = qe - qs
        ii = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 4)]))
        hh = rng.integers(0, cfg.Hq, ii.size)
        rows = np.stack([np.zeros_like(ii), hh, ii], axis=1)
        ro, rl = oracle.attention_rows(q[qs:qe].unsqueeze(0), k[ks:ke].unsqueeze(0), v[ks:ke].unsqueeze(0),
                                       cfg.causal, cfg.scale, rows)
        assert_close(o[qs + ii, hh], ro, 1e-2, "O (sequence %d, sampled rows)" % b)
        assert_close(lse[hh, qs + ii], rl, 1e-3, "LSE (sequence %d, sampled rows)" % b)
    # every row and head of the sequence with the shortest cached prefix
    b = int(np.argmin(k_lens.numpy()))
    qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
    _say("  sequence %d in full: %d queries on %d keys" % (b, qe - qs, ke - ks))
    ro, rl = oracle.attention(q[qs:qe].unsqueeze(0), k[ks:ke].unsqueeze(0), v[ks:ke].unsqueeze(0), cfg.causal,
                              cfg.scale)
    assert_close(o[qs:qe].unsqueeze(0), ro, 1e-2, "O (sequence %d, every row)" % b)
    assert_close(lse[:, qs:qe].unsqueeze(0), rl, 1e-3, "LSE (sequence %d, every row)" % b)


# ------------------------------------------------------------- determinism

def _same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_decode_is_deterministic():
    """Five decode launches on the same inputs give the same O and LSE bit for
    bit (each piece's partial result has one writer and the merge folds the
    pieces in a fixed order)."""
    lens = [1, 700, 5000, 0, 12000]
    q, kc, vc, cu = inputs.decode_inputs(lens, 64, 8, 128, torch.bfloat16, seed=41)
    qd, kd, vd, cd = q.cuda(), kc.cuda(), vc.cuda(), cu.cuda()
    runs = []
    for _ in range(5):
        o, lse = binding.decode(qd, kd, vd, cd, max(lens), inputs.fp32_scale(128))
        runs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    for o, lse in runs[1:]:
        assert _same_bits(o, runs[0][0]) and _same_bits(lse, runs[0][1])


def test_paged_decode_is_deterministic():
    """Five paged launches (appending the same rows at the same positions)
    give the same O, LSE and pages bit for bit."""
    lens = [0, 31, 64, 3000, 9000]
    x = inputs.paged_decode_inputs(lens, 64, 8, 128, 64, torch.bfloat16, seed=42)
    runs = [gpu_decode_paged(x, inputs.fp32_scale(128)) for _ in range(5)]
    for r in runs[1:]:
        assert all(_same_bits(a, b) for a, b in zip(r, runs[0]))


def test_varlen_prefill_is_deterministic():
    q_lens, k_lens = (1, 500, 2048, 0, 777), (300, 500, 6000, 64, 777)
    q, k, v, cu_q, cu_k = inputs.varlen_inputs(list(q_lens), list(k_lens), 16, 2, 128, torch.bfloat16, seed=43)
    args = (q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max(q_lens), max(k_lens), True,
            inputs.fp32_scale(128))
    runs = []
    for _ in range(5):
        o, lse = binding.fwd_varlen(*args)
        runs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    for o, lse in runs[1:]:
        assert _same_bits(o, runs[0][0]) and _same_bits(lse, runs[0][1])

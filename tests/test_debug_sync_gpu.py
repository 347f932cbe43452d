"""Race check of the kernels' pipelines: the FA_DEBUG_SYNC build of the
library (libfa_debug.so: every buffer->LDS copy waited for as soon as it is
issued, every workgroup barrier a full drain of the wave's memory operations,
register-staged tiles stored behind a barrier) runs the same arithmetic
instruction for instruction, so on the same inputs it must give the fast
build's results bit for bit.  A wait that is missing or too short in a fast
pipeline (a tile read before its copy lands, a stage overwritten while
another wave still reads it) would show as a difference.

Each case runs through both builds in this process (each build holds its own
copy of every kernel); the shapes pick every workgroup size the prefill
launch chooses and the paths of the other entry points."""
import contextlib

import pytest
import torch

from exact_io_aware_fa_amd import binding, inputs
from exact_io_aware_fa_amd import build as fa_build

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def debug_lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.load_library()
    return binding.open_library(fa_build.DEBUG_LIB)


@contextlib.contextmanager
def _using(lib):
    fast = binding.load_library()
    binding._lib = lib
    try:
        yield
    finally:
        binding._lib = fast


def _both(debug_lib, fn):
    """fn() through the fast build, then through the debug build (CPU copies)."""
    fast = [t.cpu() for t in fn()]
    torch.cuda.synchronize()
    with _using(debug_lib):
        slow = [t.cpu() for t in fn()]
        torch.cuda.synchronize()
    return fast, slow


def _same_bits(fast, slow, what):
    for i, (a, b) in enumerate(zip(fast, slow)):
        assert a.shape == b.shape and a.dtype == b.dtype, (what, i)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
            "%s: output %d differs between the fast and the FA_DEBUG_SYNC build" % (what, i)


@pytest.mark.parametrize("d,B,Hq,Hkv,N,causal", [
    (128, 1, 64, 8, 1536, True),     # 384-row workgroups (256 tiles)
    (128, 1, 64, 8, 1000, False),
    (128, 1, 8, 2, 1000, True),      # 128-row workgroups (few tiles)
    (64, 4, 16, 16, 700, False),     # 256-row workgroups
    (64, 2, 8, 4, 1100, True),       # 128-row workgroups
    (64, 1, 2, 1, 4200, True),       # 384-row workgroups at head dim 64
])
def test_prefill_matches_debug_build(debug_lib, d, B, Hq, Hkv, N, causal):
    q, k, v = inputs.prefill_inputs(B, N, N, Hq, Hkv, d, torch.bfloat16, seed=41 + d + causal)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = inputs.fp32_scale(d)
    fast, slow = _both(debug_lib, lambda: binding.fwd(qd, kd, vd, causal, scale))
    _same_bits(fast, slow, "prefill d=%d B=%d Hq=%d N=%d causal=%d" % (d, B, Hq, N, causal))


def test_varlen_prefill_matches_debug_build(debug_lib):
    q_lens, k_lens = [300, 0, 1, 777, 2048, 129], [300, 5, 0, 1500, 2048, 2000]
    for d in (64, 128):
        q, k, v, cu_q, cu_k = inputs.varlen_inputs(q_lens, k_lens, 16, 4, d, torch.bfloat16, seed=43 + d)
        qd, kd, vd, cqd, ckd = q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda()
        scale = inputs.fp32_scale(d)
        fast, slow = _both(debug_lib, lambda: binding.fwd_varlen(qd, kd, vd, cqd, ckd, max(q_lens), max(k_lens),
                                                                 True, scale))
        _same_bits(fast, slow, "varlen prefill d=%d" % d)


def test_decode_matches_debug_build(debug_lib):
    lens = [512, 1, 0, 4097, 20000, 33]
    q, kc, vc, cu = inputs.decode_inputs(lens, 64, 8, 128, torch.bfloat16, seed=44)
    qd, kd, vd, cud = q.cuda(), kc.cuda(), vc.cuda(), cu.cuda()
    scale = inputs.fp32_scale(128)
    fast, slow = _both(debug_lib, lambda: binding.decode(qd, kd, vd, cud, max(lens), scale))
    _same_bits(fast, slow, "decode")


def test_paged_decode_matches_debug_build(debug_lib):
    lens = [511, 0, 4096, 1000, 64]
    x = inputs.paged_decode_inputs(lens, 16, 2, 128, 64, torch.bfloat16, seed=45)
    scale = inputs.fp32_scale(128)
    table, seqlens = x["block_table"].cuda(), x["seqlens"].cuda()
    kn, vn = x["k_new"].cuda(), x["v_new"].cuda()

    def run():
        kp, vp = x["k_pages"].cuda(), x["v_pages"].cuda()       # fresh pages: the call appends
        o, lse = binding.decode_paged(x["q"].cuda(), kp, vp, table, seqlens, max(lens), scale, kn, vn)
        return o, lse, kp, vp

    fast, slow = _both(debug_lib, run)
    _same_bits(fast, slow, "paged decode")


@pytest.mark.parametrize("d,B,Hq,Hkv,N,causal", [
    (128, 1, 16, 2, 2048, True),
    (128, 2, 8, 2, 700, False),
    (64, 1, 8, 8, 1000, True),
])
def test_backward_matches_debug_build(debug_lib, d, B, Hq, Hkv, N, causal):
    q, k, v = inputs.prefill_inputs(B, N, N, Hq, Hkv, d, torch.bfloat16, seed=46 + d)
    g = torch.Generator().manual_seed(47 + d)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    scale = inputs.fp32_scale(d)
    o, lse = binding.fwd(qd, kd, vd, causal, scale)
    fast, slow = _both(debug_lib, lambda: binding.bwd(qd, kd, vd, o, lse, dod, causal, scale))
    _same_bits(fast, slow, "backward d=%d B=%d Hq=%d N=%d causal=%d" % (d, B, Hq, N, causal))

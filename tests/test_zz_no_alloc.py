"""fa_decode_noalloc (the decode entry point that allocates nothing: its
partial results live in the library's static device array) against fa_decode
with a caller-owned workspace, through the C ABI.

Two calls in a row, the second with a smaller input: each must give O and LSE
identical, bit for bit, to fa_decode on the same inputs (same kernels and
plan), match the fp64 oracle within the bf16 tolerances (O 1e-2, LSE 1e-3),
and leave torch's device allocation unchanged (outputs are passed in).
"""
import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import binding, inputs
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _case(q, kc, vc, cu, max_len, scale):
    qd, kd, vd, cd = q.cuda(), kc.cuda(), vc.cuda(), cu.cuda()
    o_ref, l_ref = binding.decode(qd, kd, vd, cd, max_len, scale)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    binding.decode_noalloc(qd, kd, vd, cd, max_len, scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))
    ro, rl = oracle.decode(q, kc, vc, cu, scale)
    err_o = float(np.abs(o.cpu().double().numpy() - ro).max())
    lg = lse.cpu().double().numpy()
    same_inf = np.isinf(lg) & np.isinf(rl)
    with np.errstate(invalid="ignore"):
        err_l = float(np.where(same_inf, 0.0, np.abs(lg - rl)).max())
    print("  max|dO| %.3g  max|dLSE| %.3g" % (err_o, err_l), flush=True)
    assert err_o <= 1e-2 and err_l <= 1e-3


def test_decode_noalloc_matches_decode_on_two_calls():
    cfg = inputs.DECODE_VARLEN_BF16
    print("case: decode_noalloc, the decode workload (%d sequences)" % cfg.B, flush=True)
    q, kc, vc, cu, lens = inputs.decode_config_inputs(cfg)
    _case(q, kc, vc, cu, int(lens.max()), cfg.scale)
    print("case: decode_noalloc, a smaller call after it", flush=True)
    lens = [1, 300, 0, 2049]
    q, kc, vc, cu = inputs.decode_inputs(lens, 16, 2, 64, torch.bfloat16, seed=51)
    _case(q, kc, vc, cu, max(lens), inputs.fp32_scale(64))

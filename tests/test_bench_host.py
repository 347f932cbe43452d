"""Host-side logic of bench.py (CPU only): the algorithmic counts it divides
by, and the attribution of counter dispatches to the parts of a launch."""
import torch

import bench
from exact_io_aware_fa_amd import inputs


def test_prefill_flops_is_the_causal_half():
    cfg = inputs.LLAMA70B_GQA_BF16
    assert bench.prefill_flops(cfg) == 2 ** 40


def test_varlen_flops_counts_visible_pairs():
    cfg = inputs.VarlenConfig("t", torch.bfloat16, 2, 2, 1, 8, True, 3, 0, 0)
    # sequence 0: 3 queries on 5 keys (each sees 3, 4, 5); sequence 1: 2 on 1 (0, 1)
    pairs = (3 + 4 + 5) + (0 + 1)
    assert bench.varlen_flops(cfg, torch.tensor([3, 2]), torch.tensor([5, 1])) == 4.0 * 8 * 2 * pairs


def test_paged_decode_bytes():
    cfg = inputs.DecodeConfig("t", torch.bfloat16, 2, 4, 2, 8, 1, 100)
    lens = torch.tensor([63, 64])
    row = 2 * 8 * 2
    expect = 2 * 127 * row + 4 * 2 * row + 2 * 2 * 4 * 8 * 2 + 2 * 4 * 4 + 2 * 4 + (1 + 2) * 4
    assert bench.paged_decode_bytes(cfg, lens, 64) == expect


def test_counter_dispatches_follow_the_launch_order():
    k = lambda s: "void fa::(anonymous namespace)::%s(int)" % s
    disp = {1: ("__amd_rocclr_copyBuffer", 1.0), 2: (k("prefill_bf16_kernel<128, true, false>"), 5.0),
            3: (k("decode_split_kernel<128, false>"), 7.0), 4: (k("decode_combine_kernel<128>"), 1.0),
            5: (k("paged_prep_kernel<128>"), 0.5), 6: (k("decode_split_kernel<128, true>"), 7.0),
            7: (k("decode_combine_kernel<128>"), 1.0), 8: (k("bwd_pre_kernel<128>"), 2.0),
            9: (k("bwd_dq_kernel<128, true, 4, 2>"), 3.0), 10: (k("bwd_dkdv_kernel<128, true, 8, 1>"), 4.0)}
    parts = bench._part_of_dispatches(disp)
    assert 1 not in parts
    assert [parts[i] for i in range(2, 11)] == ["prefill", "decode", "decode", "decode_paged", "decode_paged",
                                                "decode_paged", "backward", "backward", "backward"]

"""Host-side logic of bench.py (CPU only): the algorithmic counts it divides
by, and the attribution of counter dispatches to the parts of a launch."""
import os
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
            3: (k("prefill_bf16_kernel<128, true, true>"), 6.0),
            4: (k("decode_split_kernel<128, false>"), 7.0), 5: (k("decode_combine_kernel<128>"), 1.0),
            6: (k("paged_prep_kernel<128>"), 0.5), 7: (k("decode_split_kernel<128, true>"), 7.0),
            8: (k("decode_combine_kernel<128>"), 1.0), 9: (k("bwd_pre_kernel<128>"), 2.0),
            10: (k("bwd_dq_kernel<128, true, 4, 2>"), 3.0), 11: (k("bwd_dkdv_kernel<128, true, 8, 1>"), 4.0)}
    parts = bench._part_of_dispatches(disp)
    assert 1 not in parts
    assert [parts[i] for i in range(2, 12)] == ["prefill", "varlen_prefill", "decode", "decode", "decode_paged",
                                                "decode_paged", "decode_paged", "backward", "backward", "backward"]


def test_varlen_prefill_bytes():
    cfg = inputs.VarlenConfig("t", torch.bfloat16, 2, 4, 2, 8, True, 3, 0, 0)
    q_lens, k_lens = torch.tensor([3, 2]), torch.tensor([5, 1])
    # Q and O: 5 rows x 4 heads x 8 x 2 B each; K and V: 6 rows x 2 heads x 8 x 2 B each;
    # LSE: 5 x 4 floats; two offset arrays of 3 int32
    expect = 2 * 5 * 4 * 8 * 2 + 2 * 6 * 2 * 8 * 2 + 5 * 4 * 4 + 2 * 3 * 4
    assert bench.varlen_prefill_bytes(cfg, q_lens, k_lens) == expect


def test_mfma_summary_sums_each_part(tmp_path, monkeypatch):
    """Busy cycles over (SIMDs x duration x clock), and MOPS x 512 as flops,
    summed over the kernels of a part; the file it writes carries digests."""
    k = lambda s: "void fa::(anonymous namespace)::%s(int)" % s
    rows = [(1, "__amd_rocclr_copyBuffer", 0, 1000, 0.0, 0.0),
            (2, k("prefill_bf16_kernel<128, true, false>"), 0, 1000, 1.2e6, 2.4e6),
            (3, k("bwd_pre_kernel<128>"), 0, 500, 0.0, 0.0),
            (4, k("bwd_dq_kernel<128, true, 4, 2>"), 0, 1000, 0.6e6, 1.2e6),
            (5, k("bwd_dkdv_kernel<128, true, 8, 1>"), 0, 2000, 0.6e6, 1.2e6)]
    path = tmp_path / "c.csv"
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
        for did, name, t0, t1, busy, mops in rows:
            for cn, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops),
                          ("GRBM_GUI_ACTIVE", 1.0)):
                f.write('%d,"%s","%s",%r,%d,%d\n' % (did, name, cn, v, t0, t1))
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "mfma.json"))
    out = bench.mfma_summary(str(path), n_simd=1000, clock_ghz=2.0)
    # prefill: 1.2e6 busy cycles / 1000 SIMDs over 1 us at 2 GHz = 2000 cycles
    assert abs(out["prefill"]["mfma_busy"] - 0.6) < 1e-9
    assert out["prefill"]["bf16_mfma_flops"] == 2.4e6 * 512
    # backward: 1.2e6 / 1000 over 3.5 us at 2 GHz
    assert abs(out["backward"]["mfma_busy"] - round(1200.0 / 7000.0, 4)) < 1e-9
    assert [x["kernel"] for x in out["backward"]["kernels"]] == ["bwd_pre_kernel", "bwd_dq_kernel",
                                                                 "bwd_dkdv_kernel"]
    assert out["decode"]["bf16_mfma_flops"] == 0.0
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "mfma.json"))
    assert bench.measured_mfma_flops("backward") == 2.4e6 * 512


def test_small_prefill_bytes_and_floors():
    """Algorithmic bytes of the three small workloads: Q, K, V read once, O and
    LSE written once, and the HBM floor of the bf16 ones at 8 TB/s."""
    c1, c2, c3 = inputs.SINGLE_HEAD_F32, inputs.BERT_LARGE_BF16, inputs.GPT2_CAUSAL_BF16
    assert bench.prefill_bytes(c1, 4) == 4 * 256 * 64 * 4 + 256 * 4 == 263168
    assert bench.prefill_bytes(c2, 2) == 4 * 16 * 512 * 16 * 64 * 2 + 16 * 16 * 512 * 4 == 67633152
    assert bench.prefill_bytes(c3, 2) == 4 * 8 * 1024 * 12 * 64 * 2 + 8 * 12 * 1024 * 4 == 50724864
    e2 = bench.small_prefill_entry(c2, 0.0169, 5)
    assert e2["bound"] == "hbm" and e2["hbm_floor_us"] == 8.45
    assert abs(e2["frac"] - 67633152 / 0.0169e-3 / 8e12) < 1e-4
    assert abs(e2["frac_mfma"] - 2 ** 34 / 0.0169e-3 / 2.5e15) < 1e-4
    e1 = bench.small_prefill_entry(c1, 0.04, 1)
    assert e1["bound"] == "alu" and e1["peak"] == 157.3


def test_small_prefill_copies_exceed_the_infinity_cache():
    """The rotated input copies of each bf16 workload together exceed 256 MB."""
    for key, attr, copies in bench.SMALL_PREFILL:
        cfg = getattr(inputs, attr)
        if cfg.dtype == torch.bfloat16:
            assert copies * bench.prefill_bytes(cfg, 2) > 256 * 2 ** 20, key


def test_more_than_one_gpu_is_refused():
    """The bench measures one GPU: --gpus other than 1 exits with status 2 and
    a message before anything touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

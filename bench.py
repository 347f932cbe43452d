#!/usr/bin/env python3
"""Benchmark of the exact attention forward hot path on one MI355X.

One step = the whole hot path over one batch of synthetic inputs:
  * prefill: causal GQA attention, B=1, Hq=64, Hkv=8, N=Nk=8192, d=128, bf16
    (Llama2-70B-shaped), through fa_fwd;
  * decode: one query token for each of 32 sequences against a packed bf16 KV
    cache with lengths drawn uniform on 512..32768 (seed 0), Hq=64, Hkv=8,
    d=128, through fa_decode.
Inputs are generated once (seeded) and are resident in HBM before timing.

Prints one JSON line.  `value` is the prefill throughput in TFLOP/s counted as
4*B*Hq*N*Nk*d/2 (the causal half), measured with HIP events around each
launch on the launch stream; the decode part is reported beside it in GB/s of
algorithmic bytes (K and V cache, q, o, lse and cu_seqlens, each once).
Every part below runs W times untimed before any part is timed (the chip's
clocks settle only after some tens of ms of load).  After the timed steps, a
chunked variable-length prefill (16 sequences of
2048-token chunks on caches of 0..14336 earlier tokens, fa_fwd_varlen) is timed
on its own and reported as `roofline_varlen_prefill`, counting 4*d*Hq flops
per visible (query, key) pair.  Then the decode workload on a paged cache of
64-row blocks, with each sequence's new K/V row appended in the same call
(fa_decode_paged), is timed and reported as `roofline_decode_paged` in GB/s of
algorithmic bytes (the cached rows, the new rows read and written, q, o, lse,
the lengths and the block-table entries used, each once).  Last, the backward
of the prefill workload (fa_bwd, given the forward's O and LSE and a seeded
dO) is timed and reported as `roofline_backward`, counting the five products
of the chain rule (S recomputed, dP, dV, dK, dQ: 2.5 times the forward's
flops); the kernels compute S and dP twice (seven products), which the count
leaves out.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --pmc-pass      # a copy of known size, then one launch of each part
                                    # (prefill, decode, paged decode, backward), for
                                    # rocprofv3 counter collection
    python bench.py --traffic-summary FETCH.csv WRITE.csv
                                    # counters of two such passes -> profiles/traffic.json
    python bench.py --mfma-summary MFMA.csv
                                    # MFMA busy fraction and executed bf16 MFMA flops per
                                    # part, from one pass of SQ_VALU_MFMA_BUSY_CYCLES,
                                    # GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E peak
METRIC = ("attention fwd TFLOP/s & % bf16 MFMA peak (prefill); "
          "GB/s & % HBM peak (decode)")
_CSRC = "exact_io_aware_fa_amd/csrc/"
# sources whose change invalidates a kernel's measured traffic
TRAFFIC_SOURCES = {
    "prefill": [_CSRC + "fa_prefill_bf16.hip", _CSRC + "fa_common.h"],
    "varlen_prefill": [_CSRC + "fa_prefill_bf16.hip", _CSRC + "fa_common.h"],
    "decode": [_CSRC + "fa_decode.hip", _CSRC + "fa_common.h", _CSRC + "fa_api.cpp"],
    "decode_paged": [_CSRC + "fa_decode.hip", _CSRC + "fa_common.h", _CSRC + "fa_api.cpp"],
    "backward": [_CSRC + "fa_bwd_bf16.hip", _CSRC + "fa_common.h"],
}
# Kernels of each part: the kernel-name fragment of the part's first launch,
# and the fragments of all its kernels.  The counter pass launches the parts
# one after the other, so a dispatch belongs to the last part started before
# it (the paged decode reuses the decode's kernel names; the varlen prefill's
# name also holds the prefill's fragment, so it comes later in this table).
TRAFFIC_KERNELS = {
    "prefill": ("prefill_bf16_kernel", ["prefill_bf16_kernel"]),
    "varlen_prefill": ("prefill_bf16_kernel<128, true, true", ["prefill_bf16_kernel"]),
    "decode": ("decode_split_kernel<128, false>", ["decode_split_kernel", "decode_combine_kernel"]),
    "decode_paged": ("paged_prep_kernel", ["paged_prep_kernel", "decode_split_kernel", "decode_combine_kernel"]),
    "backward": ("bwd_pre_kernel", ["bwd_pre_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel"]),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")
PMC_COPY_BYTES = 1 << 30           # calibration copy: 1 GiB read + 1 GiB written


def source_digest(path):
    """Digest of a source's code: comments and whitespace removed, so that an
    edit of the comments alone keeps a measurement valid."""
    import re
    with open(os.path.join(ROOT, path)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(part):
    """HBM bytes per launch of `part` from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[part]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources") != {p: source_digest(p) for p in TRAFFIC_SOURCES[part]}:
        return None
    return rec.get("hbm_bytes_per_launch")


def measured_mfma_flops(part):
    """bf16 MFMA flops executed per launch of `part` (masked and recomputed
    work included) from the committed counter summary, or None when there is
    none or the kernel sources changed since it was taken."""
    try:
        with open(MFMA_FILE) as f:
            rec = json.load(f)[part]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources") != {p: source_digest(p) for p in TRAFFIC_SOURCES[part]}:
        return None
    return rec.get("bf16_mfma_flops_per_launch")


def _counter_per_dispatch(csv_path, counter):
    """{dispatch id (int): (kernel name, value summed over the counter's instances)}"""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            did = int(r["Dispatch_Id"])
            name, val = out.get(did, (r["Kernel_Name"], 0.0))
            out[did] = (name, val + float(r["Counter_Value"]))
    return out


def _part_of_dispatches(disp):
    """{dispatch id: part} following the launch order of the counter pass."""
    parts, cur = {}, None
    for did in sorted(disp):
        name = disp[did][0]
        for part, (start, _) in TRAFFIC_KERNELS.items():
            if start in name:
                cur = part
        if cur is not None and any(fr in name for fr in TRAFFIC_KERNELS[cur][1]):
            parts[did] = cur
    return parts


def traffic_summary(fetch_csv, write_csv):
    """HBM traffic per launch from two rocprofv3 counter passes over
    `bench.py --pmc-pass` (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch).
    Each counter is scaled by what it reads for the pass's 1 GiB device copy
    (the largest copy dispatch), then summed over the kernels of one launch.
    Writes profiles/traffic.json (with digests of the kernel sources) and
    prints the figures."""
    result = {}
    factors = {}
    per_part = {part: {} for part in TRAFFIC_KERNELS}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _counter_per_dispatch(path, counter)
        copies = [v for n, v in disp.values() if "copyBuffer" in n]
        factor = PMC_COPY_BYTES / (max(copies) * 1024.0)
        factors[counter] = factor
        owner = _part_of_dispatches(disp)
        for part in TRAFFIC_KERNELS:
            per_part[part][counter] = sum(v * 1024.0 * factor for did, (n, v) in disp.items()
                                          if owner.get(did) == part)
    for part, c in per_part.items():
        result[part] = {"fetch_bytes_per_launch": round(c["FETCH_SIZE"]),
                        "write_bytes_per_launch": round(c["WRITE_SIZE"]),
                        "hbm_bytes_per_launch": round(c["FETCH_SIZE"] + c["WRITE_SIZE"]),
                        "sources": {p: source_digest(p) for p in TRAFFIC_SOURCES[part]}}
    result["calibration"] = {"copy_bytes": PMC_COPY_BYTES, "fetch_factor": round(factors["FETCH_SIZE"], 4),
                             "write_factor": round(factors["WRITE_SIZE"], 4)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(result, indent=1, sort_keys=True))


def mfma_summary(csv_path, n_simd=1024, clock_ghz=2.4):
    """MFMA use per part of a counter pass over `bench.py --pmc-pass`.

    SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) divided by the SIMD
    count (256 CUs x 4) is how many cycles each SIMD's matrix unit was busy;
    over the dispatch's own duration (its trace timestamps) at the 2.4 GHz
    peak clock that is the MFMA utilisation against the dense peak.
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 is the bf16 MFMA flops executed,
    masked-away work included.  GRBM_GUI_ACTIVE is not used as the
    denominator: the pass reports it summed over the XCDs and over a counter
    window wider than the dispatch.  Writes the executed flops per launch
    (with digests of the kernel sources) to profiles/mfma.json and prints the
    figures."""
    import csv
    disp = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            name = r["Kernel_Name"]
            e = disp.setdefault(did, {"name": name, "vals": {},
                                      "dur_s": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
            e["vals"][r["Counter_Name"]] = e["vals"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    owner = _part_of_dispatches({d: (e["name"], 0.0) for d, e in disp.items()})

    def short(name):
        name = name.split("(")[0] if "(anonymous" not in name else name.split("::")[-1]
        return name.split("<")[0].split("(")[0].strip()

    out = {"clock_ghz": clock_ghz, "n_simd": n_simd}
    for part in TRAFFIC_KERNELS:
        tot_busy = tot_flops = tot_dur = 0.0
        kernels = []
        for did, e in sorted(disp.items()):
            if owner.get(did) != part:
                continue
            busy = e["vals"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            flops = e["vals"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
            tot_busy += busy
            tot_flops += flops
            tot_dur += e["dur_s"]
            kernels.append({"kernel": short(e["name"]), "us": round(e["dur_s"] * 1e6, 1),
                            "mfma_busy": round(busy / n_simd / (e["dur_s"] * clock_ghz * 1e9), 4),
                            "bf16_mfma_flops": flops,
                            "tflops_executed": round(flops / e["dur_s"] / 1e12, 1)})
        out[part] = {"us": round(tot_dur * 1e6, 1), "mfma_busy_cycles": tot_busy,
                     "mfma_busy": round(tot_busy / n_simd / max(1e-12, tot_dur * clock_ghz * 1e9), 4),
                     "bf16_mfma_flops": tot_flops,
                     "tflops_executed": round(tot_flops / max(1e-12, tot_dur) / 1e12, 1),
                     "kernels": kernels}
    rec = {part: {"bf16_mfma_flops_per_launch": out[part]["bf16_mfma_flops"],
                  "mfma_busy_cycles_per_launch": out[part]["mfma_busy_cycles"],
                  "sources": {p: source_digest(p) for p in TRAFFIC_SOURCES[part]}}
           for part in TRAFFIC_KERNELS}
    with open(MFMA_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return out


def prefill_flops(cfg):
    f = 4.0 * cfg.B * cfg.Hq * cfg.N * cfg.Nk * cfg.d
    return f / 2 if cfg.causal else f


def varlen_prefill_bytes(cfg, q_lens, k_lens):
    """Algorithmic bytes of one packed varlen prefill: Q, K, V read once, O and
    LSE written once, the two offset arrays read once."""
    sq, sk = int(q_lens.sum()), int(k_lens.sum())
    qo = 2 * sq * cfg.Hq * cfg.d * 2
    kv = 2 * sk * cfg.Hkv * cfg.d * 2
    return qo + kv + sq * cfg.Hq * 4 + 2 * (cfg.B + 1) * 4


def decode_bytes(cfg, total_len):
    kv = 2 * total_len * cfg.Hkv * cfg.d * 2
    qo = 2 * cfg.B * cfg.Hq * cfg.d * 2
    return kv + qo + cfg.B * cfg.Hq * 4 + (cfg.B + 1) * 4


PAGED_BLOCK = 64                   # rows per block of the paged decode workload


def paged_decode_bytes(cfg, lens, block_size):
    """Algorithmic bytes of one paged decode step with the new rows appended."""
    row = cfg.Hkv * cfg.d * 2                      # one K (or V) row of all kv heads, bf16
    total = int(lens.sum())
    blocks = sum((int(L) + 1 + block_size - 1) // block_size for L in lens.tolist())
    return (2 * total * row + 2 * 2 * cfg.B * row + 2 * cfg.B * cfg.Hq * cfg.d * 2 + cfg.B * cfg.Hq * 4
            + cfg.B * 4 + blocks * 4)



FP32_VALU_PEAK_TFLOPS = 157.3      # MI355X fp32 vector peak (256 CUs x 256 flop/clk x 2.4 GHz)
# The three small prefill workloads, each timed on rotated input copies whose
# total size exceeds the 256 MB Infinity Cache, so that every launch reads its
# inputs from HBM (the configs' algorithmic bytes are 0.26 MB, 68 MB, 51 MB).
SMALL_PREFILL = (("single_head_fp32", "SINGLE_HEAD_F32", 1),
                 ("bert_large_bf16", "BERT_LARGE_BF16", 5),
                 ("gpt2_causal_bf16", "GPT2_CAUSAL_BF16", 6))


def prefill_bytes(cfg, elem_bytes):
    """Algorithmic bytes of one prefill launch: Q, K, V read once, O and LSE
    (fp32) written once."""
    qo = 2 * cfg.B * cfg.N * cfg.Hq * cfg.d * elem_bytes
    kv = 2 * cfg.B * cfg.Nk * cfg.Hkv * cfg.d * elem_bytes
    return qo + kv + cfg.B * cfg.Hq * cfg.N * 4


def device_info(torch):
    """The GPU's own figures, and the peaks derived from them: bf16 dense MFMA
    = CUs x peak clock x 4096 flop/clk/CU; HBM = memory clock x 4 x bus width
    / 8.  The factor 4: this part's HBM3E pins carry 8 Gb/s at the 2 GHz
    memory clock the device reports (with 2 transfers per clock the 8192-bit
    bus would peak at 4.1 TB/s, below what the decode alone measures)."""
    pr = torch.cuda.get_device_properties(0)
    cus, clk_khz = int(pr.multi_processor_count), int(getattr(pr, "clock_rate", 0))
    mem_khz, bus = int(getattr(pr, "memory_clock_rate", 0)), int(getattr(pr, "memory_bus_width", 0))
    if not (clk_khz and mem_khz and bus):
        # torch leaves these at 0 on ROCm: ask HIP (hipDeviceGetAttribute with the
        # HIP 7 enum values of ClockRate, MemoryClockRate, MemoryBusWidth)
        import ctypes
        try:
            hip = ctypes.CDLL("libamdhip64.so")
            val = ctypes.c_int()
            got = {}
            for name, attr in (("clk", 5), ("mem", 60), ("bus", 59)):
                got[name] = val.value if hip.hipDeviceGetAttribute(ctypes.byref(val), attr, 0) == 0 else 0
            clk_khz, mem_khz, bus = got["clk"] or clk_khz, got["mem"] or mem_khz, got["bus"] or bus
        except OSError:
            pass
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "cus": cus, "clock_mhz": clk_khz / 1000.0,
            "memory_clock_mhz": mem_khz / 1000.0, "memory_bus_width_bits": bus,
            "peak_bf16_tflops_derived": round(cus * clk_khz * 1e3 * 4096 / 1e12, 1),
            "peak_hbm_gbs_derived": round(mem_khz * 1e3 * 4 * bus / 8 / 1e9, 1),
            "peak_bf16_tflops_spec": MFMA_BF16_PEAK_TFLOPS, "peak_hbm_gbs_spec": HBM_PEAK_GBS}


def time_small_prefill(torch, binding, inputs, dev, cfg, copies, steps, warmup):
    """Mean launch time (ms) of fa_fwd on `cfg`, each launch on the next of
    `copies` device copies of the same seeded inputs."""
    q, k, v = inputs.prefill_config_inputs(cfg)
    sets = []
    for _ in range(copies):
        qd = q.to(dev)
        sets.append((qd, k.to(dev), v.to(dev), torch.empty_like(qd),
                     torch.empty((cfg.B, cfg.Hq, cfg.N), dtype=torch.float32, device=dev)))
    for i in range(max(warmup, copies)):
        a = sets[i % copies]
        binding.fwd(a[0], a[1], a[2], cfg.causal, cfg.scale, out=a[3], lse=a[4])
    torch.cuda.synchronize()
    n = max(steps, 4 * copies)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        a = sets[i % copies]
        binding.fwd(a[0], a[1], a[2], cfg.causal, cfg.scale, out=a[3], lse=a[4])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def small_prefill_entry(cfg, ms, copies):
    """roofline object of a small prefill workload: fp32 against the vector
    ALU peak; bf16 against HBM (its intensity, 254 flop/B, is below the bf16
    ridge of about 312 flop/B) with the MFMA fraction beside it."""
    flops = prefill_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    if cfg.dtype.itemsize == 4:
        nbytes = prefill_bytes(cfg, 4)
        return {"bound": "alu", "achieved": round(tflops, 4), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP32_VALU_PEAK_TFLOPS, 5), "traffic": None, "ms": round(ms, 5),
                "flops_per_launch": flops, "bytes_per_launch": nbytes,
                "note": "one launch of one 256-row head: bound by the launch and a few memory round trips, not by the ALU"}
    nbytes = prefill_bytes(cfg, 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "ms": round(ms, 5),
            "hbm_floor_us": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
            "tflops": round(tflops, 1), "frac_mfma": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": flops, "bytes_per_launch": nbytes, "input_copies": copies}


def varlen_flops(cfg, q_lens, k_lens):
    """4*d*Hq per visible (query, key) pair; causal is bottom-right per sequence."""
    pairs = 0
    for n, nk in zip(q_lens.tolist(), k_lens.tolist()):
        if not cfg.causal:
            pairs += n * nk
        else:
            # query i sees keys 0 .. i + nk - n (clipped to 0 .. nk - 1)
            pairs += sum(max(0, min(nk, i + nk - n + 1)) for i in range(n))
    return 4.0 * cfg.d * cfg.Hq * pairs


def cpu_baseline(q, k, v, cfg):
    """The fp64 oracle on a bounded sample of the prefill workload: every 8th
    query row, all heads.  Reported as algorithmic TFLOP/s of the sample."""
    import numpy as np
    from oracle import oracle
    rows = np.array([(0, h, i) for i in range(0, cfg.N, 8) for h in range(cfg.Hq)])
    visible = (rows[:, 2] + 1 + (cfg.Nk - cfg.N)) if cfg.causal else np.full(len(rows), cfg.Nk)
    flops = float((4.0 * cfg.d * visible).sum())
    threads = oracle.DEFAULT_THREADS
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, cfg.causal, cfg.scale, rows, nthreads=threads)
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "sample": "%d query rows (every 8th row x %d heads) of the prefill workload, "
                      "%.1f s wall; threads = the CPUs this process may use, capped at 16 "
                      "(the host share of one GPU)" % (len(rows), cfg.Hq, dt)}


def setup_varlen(torch, binding, inputs, dev):
    """The chunked varlen prefill workload resident on the device: returns
    (launch, config, query lengths, key lengths)."""
    vcfg = inputs.VARLEN_CHUNKED_BF16
    vq, vk, vv, vcu_q, vcu_k, vq_lens, vk_lens = inputs.varlen_config_inputs(vcfg)
    vqd, vkd, vvd = vq.to(dev), vk.to(dev), vv.to(dev)
    vcuq, vcuk = vcu_q.to(dev), vcu_k.to(dev)
    del vq, vk, vv
    vo = torch.empty_like(vqd)
    vl = torch.empty((vcfg.Hq, vqd.shape[0]), dtype=torch.float32, device=dev)
    vmax_q, vmax_k = int(vq_lens.max()), int(vk_lens.max())

    def varlen():
        binding.fwd_varlen(vqd, vkd, vvd, vcuq, vcuk, vmax_q, vmax_k, vcfg.causal, vcfg.scale, out=vo, lse=vl)

    return varlen, vcfg, vq_lens, vk_lens


def setup_paged(torch, binding, inputs, dcfg, dev, max_len):
    """The decode workload on a paged cache of PAGED_BLOCK-row blocks with the
    new rows appended: returns the launch closure."""
    px = inputs.paged_config_inputs(dcfg, PAGED_BLOCK)
    t = {n: px[n].to(dev) for n in ("q", "k_new", "v_new", "k_pages", "v_pages", "block_table", "seqlens")}
    del px
    t["o"] = torch.empty_like(t["q"])
    t["lse"] = torch.empty((dcfg.B, dcfg.Hq), dtype=torch.float32, device=dev)
    t["ws"] = torch.empty(max(1, binding.decode_paged_workspace_bytes(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.d, max_len)),
                          dtype=torch.uint8, device=dev)

    def paged():
        # the same rows are appended at the same positions on every call
        binding.decode_paged(t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["seqlens"], max_len,
                             dcfg.scale, t["k_new"], t["v_new"], out=t["o"], lse=t["lse"], workspace=t["ws"])
    return paged


def setup_backward(torch, binding, pcfg, dev, qd, kd, vd, o, lse):
    """The backward of the prefill workload for a seeded dO (o and lse must
    hold the forward's results): returns the launch closure."""
    g = torch.Generator().manual_seed(1)
    gdo = torch.randn(tuple(qd.shape), generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd))
    gws = torch.empty(max(1, int(binding.load_library().fa_bwd_workspace_bytes(pcfg.B, pcfg.Hq, pcfg.N))),
                      dtype=torch.uint8, device=dev)

    def backward():
        binding.bwd(qd, kd, vd, o, lse, gdo, pcfg.causal, pcfg.scale, dq=grads[0], dk=grads[1], dv=grads[2],
                    workspace=gws)
    return backward


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter passes into profiles/traffic.json")
    ap.add_argument("--mfma-summary", metavar="MFMA_CSV",
                    help="MFMA busy fraction and bf16 MFMA flops per part from one rocprofv3 counter pass")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU; the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_io_aware_fa_amd import binding, inputs

    binding.load_library()
    dev = torch.device("cuda:0")
    pcfg = inputs.LLAMA70B_GQA_BF16
    dcfg = inputs.DECODE_VARLEN_BF16

    q, k, v = inputs.prefill_config_inputs(pcfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((pcfg.B, pcfg.Hq, pcfg.N), dtype=torch.float32, device=dev)

    dq, kc, vc, cu, lens = inputs.decode_config_inputs(dcfg)
    max_len = int(lens.max())
    total_len = int(lens.sum())
    dqd, kcd, vcd, cud = dq.to(dev), kc.to(dev), vc.to(dev), cu.to(dev)
    del kc, vc
    do = torch.empty_like(dqd)
    dlse = torch.empty((dcfg.B, dcfg.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, binding.decode_workspace_bytes(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.d, max_len)),
                     dtype=torch.uint8, device=dev)

    def prefill():
        binding.fwd(qd, kd, vd, pcfg.causal, pcfg.scale, out=o, lse=lse)

    def decode():
        binding.decode(dqd, kcd, vcd, cud, max_len, dcfg.scale, out=do, lse=dlse, workspace=ws)

    if args.pmc_pass:
        src = torch.empty(PMC_COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        varlen = setup_varlen(torch, binding, inputs, dev)[0]
        paged = setup_paged(torch, binding, inputs, dcfg, dev, max_len)
        backward = setup_backward(torch, binding, pcfg, dev, qd, kd, vd, o, lse)
        torch.cuda.synchronize()
        dst.copy_(src)
        prefill()
        varlen()
        decode()
        paged()
        backward()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": True, "copy_bytes": PMC_COPY_BYTES}))
        return

    # Every part resident, then every part's W untimed runs, then every part
    # timed over K launches.  After idle the chip needs some tens of ms of load
    # before its clocks settle (the first prefill launches of a fresh process
    # run about 10% slower than later ones); warming all parts before timing
    # any keeps the timed regions out of that ramp.  (The backward takes the
    # forward's O and LSE, which the warm-up steps, or else the timed steps,
    # have written before it first runs.)
    varlen, vcfg, vq_lens, vk_lens = setup_varlen(torch, binding, inputs, dev)
    vmax_k = int(vk_lens.max())
    paged = setup_paged(torch, binding, inputs, dcfg, dev, max_len)
    backward = setup_backward(torch, binding, pcfg, dev, qd, kd, vd, o, lse)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        prefill()
        decode()
    for part in (varlen, paged, backward):
        for _ in range(args.warmup):
            part()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        ev[s][0].record()
        prefill()
        ev[s][1].record()
        decode()
        ev[s][2].record()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K

    flops = prefill_flops(pcfg)
    tflops = flops / (pre_avg * 1e-3) / 1e12
    dbytes = decode_bytes(dcfg, total_len)
    gbs = dbytes / (dec_avg * 1e-3) / 1e9

    def time_part(part):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            part()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    # chunked variable-length prefill
    var_ms = time_part(varlen)
    vflops = varlen_flops(vcfg, vq_lens, vk_lens)
    vtflops = vflops / (var_ms * 1e-3) / 1e12

    # the decode workload on a paged cache, new rows appended
    paged_ms = time_part(paged)
    pbytes = paged_decode_bytes(dcfg, lens, PAGED_BLOCK)
    pgbs = pbytes / (paged_ms * 1e-3) / 1e9

    # backward of the prefill workload
    bwd_ms = time_part(backward)
    bflops = 2.5 * flops
    btflops = bflops / (bwd_ms * 1e-3) / 1e12

    # the three small prefill workloads, each on rotated input copies
    del varlen, paged, backward
    small = {}
    for key, attr, copies in SMALL_PREFILL:
        scfg = getattr(inputs, attr)
        small[key] = small_prefill_entry(scfg, time_small_prefill(torch, binding, inputs, dev, scfg, copies, K,
                                                                  args.warmup), copies)
        small[key]["config"] = {"B": scfg.B, "Hq": scfg.Hq, "Hkv": scfg.Hkv, "N": scfg.N, "Nk": scfg.Nk,
                                "d": scfg.d, "causal": scfg.causal,
                                "dtype": str(scfg.dtype).replace("torch.", "")}
        torch.cuda.empty_cache()

    pre_traffic = measured_traffic("prefill")
    var_traffic = measured_traffic("varlen_prefill")
    dec_traffic = measured_traffic("decode")
    paged_traffic = measured_traffic("decode_paged")
    bwd_traffic = measured_traffic("backward")

    def mfma_use(part, ms):
        ex = measured_mfma_flops(part)
        if ex is None:
            return None
        rate = ex / (ms * 1e-3) / 1e12
        return {"executed_flops": ex, "executed_tflops": round(rate, 1),
                "frac": round(rate / MFMA_BF16_PEAK_TFLOPS, 4)}

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16)",
        "config": {
            "workload": "causal GQA prefill B1 Hq64 Hkv8 N8192 d128 + varlen KV-cache decode "
                        "32 seqs L512-32768 (sum %d) Hq64 Hkv8 d128" % total_len,
            "prefill": {"B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "N": pcfg.N, "Nk": pcfg.Nk,
                        "d": pcfg.d, "causal": pcfg.causal, "ms": round(pre_avg, 4),
                        "ms_min": round(min(pre_ms), 4), "ms_max": round(max(pre_ms), 4),
                        "flops_per_launch": flops},
            "decode": {"B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "d": dcfg.d,
                       "sum_len": total_len, "max_len": max_len, "ms": round(dec_avg, 4),
                       "ms_min": round(min(dec_ms), 4), "ms_max": round(max(dec_ms), 4),
                       "bytes_per_launch": dbytes, "GB/s": round(gbs, 1),
                       "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)},
            "varlen_prefill": {"B": vcfg.B, "Hq": vcfg.Hq, "Hkv": vcfg.Hkv, "d": vcfg.d, "causal": vcfg.causal,
                               "chunk": vcfg.chunk, "sum_q": int(vq_lens.sum()), "sum_k": int(vk_lens.sum()),
                               "max_k": vmax_k, "ms": round(var_ms, 4), "flops_per_launch": vflops},
            "decode_paged": {"B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "d": dcfg.d, "block_size": PAGED_BLOCK,
                             "appended_rows": dcfg.B, "sum_len": total_len, "ms": round(paged_ms, 4),
                             "bytes_per_launch": pbytes, "GB/s": round(pgbs, 1)},
            "backward": {"B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "N": pcfg.N, "Nk": pcfg.Nk, "d": pcfg.d,
                         "causal": pcfg.causal, "ms": round(bwd_ms, 4), "flops_per_launch": bflops},
        },
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": pre_traffic},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "traffic": dec_traffic},
        "roofline_varlen_prefill": {"bound": "mfma", "achieved": round(vtflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(vtflops / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "traffic": var_traffic},
        "roofline_decode_paged": {"bound": "hbm", "achieved": round(pgbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(pgbs / HBM_PEAK_GBS, 4), "traffic": paged_traffic},
        "roofline_backward": {"bound": "mfma", "achieved": round(btflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(btflops / MFMA_BF16_PEAK_TFLOPS, 4),
                              "traffic": bwd_traffic},
        "roofline_c1_single_head_fp32": small["single_head_fp32"],
        "roofline_c2_bert_large_bf16": small["bert_large_bf16"],
        "roofline_c3_gpt2_causal_bf16": small["gpt2_causal_bf16"],
        "device": device_info(torch),
        "mfma_util": {"prefill": mfma_use("prefill", pre_avg), "varlen_prefill": mfma_use("varlen_prefill", var_ms),
                      "decode": mfma_use("decode", dec_avg),
                      "decode_paged": mfma_use("decode_paged", paged_ms),
                      "backward": mfma_use("backward", bwd_ms)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(q, k, v, pcfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

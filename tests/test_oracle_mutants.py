"""Planted mistakes: each mutant is a copy of oracle.c with one plausible error
(compiled on the CPU into a temporary library).  The pin battery below, built
from the same independent facts as test_oracle.py (hand-worked closed forms,
the scalar brute force, torch SDPA in fp64), must reject every mutant and
accept the unmodified source.
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
from tests.test_oracle import GOLDEN, _arr

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "scale dropped": ("srow[j] = scale * dot;", "srow[j] = dot;"),
    "mask off by one": ("nvis = last < 0 ? 0 : (last + 1 > nk ? nk : (int)(last + 1));",
                        "nvis = last < 0 ? 0 : (last > nk ? nk : (int)last);"),
    "top-left causal alignment": ("int64_t last = (int64_t)i + J->Nk - J->N;",
                                  "int64_t last = (int64_t)i;"),
    "interleaved kv heads": ("const int g = h / group;", "const int g = h % J->Hkv;"),
    "K used in place of V": ("acc += prow[j] * widen(v, dtype,", "acc += prow[j] * widen(k, dtype,"),
    "base-2 LSE": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "LSE without the max": ("*lse = m + log(l);", "*lse = log(l);"),
    "unnormalised P": ("prow[j] /= l;", "prow[j] /= 1.0;"),
    "decode drops last cache row": ("nk = (int)(J->cu[b + 1] - start);",
                                    "nk = (int)(J->cu[b + 1] - start) - 1;"),
    "decode reads next sequence": ("const int64_t start = J->cu[b];",
                                   "const int64_t start = J->cu[b] + 1;"),
    "query row stride wrong": ("q_off = (((int64_t)b * J->N + i) * J->Hq + h) * J->d;",
                               "q_off = (((int64_t)b * J->Hq + h) * J->N + i) * J->d;"),
}


def _ok(a, b, tol=1e-10):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape or np.isnan(a).any() or np.isnan(b).any():
        return False
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(a - b))
    return err.max(initial=0.0) <= tol


def battery(lib):
    """Names of the pins the library fails (an error raised counts as a failure)."""
    failures = []

    def pin(name, fn):
        try:
            if not fn():
                failures.append(name)
        except Exception:
            failures.append(name)

    with open(GOLDEN) as f:
        gold = json.load(f)
    for c in gold["prefill"]:
        def golden_prefill(c=c):
            q, k, v = (torch.from_numpy(_arr(c[x])) for x in ("q", "k", "v"))
            o, lse = oracle.attention(q, k, v, c["causal"], c["scale"], lib=lib)
            return _ok(o, _arr(c["o"])) and _ok(lse, _arr(c["lse"]))
        pin("golden " + c["name"], golden_prefill)
    for c in gold["decode"]:
        def golden_decode(c=c):
            q, kc, vc = (torch.from_numpy(_arr(c[x])) for x in ("q", "k_cache", "v_cache"))
            cu = torch.tensor(c["cu_seqlens"], dtype=torch.int32)
            o, lse = oracle.decode(q, kc, vc, cu, c["scale"], lib=lib)
            return _ok(o, _arr(c["o"])) and _ok(lse, _arr(c["lse"]))
        pin("golden " + c["name"], golden_decode)

    g = torch.Generator().manual_seed(123)
    for (Hq, Hkv, N, Nk, d) in [(2, 1, 4, 7, 8), (4, 2, 6, 6, 8), (2, 2, 7, 3, 8)]:
        for causal in (False, True):
            q = torch.randn(2, N, Hq, d, generator=g, dtype=torch.float64)
            k = torch.randn(2, Nk, Hkv, d, generator=g, dtype=torch.float64)
            v = torch.randn(2, Nk, Hkv, d, generator=g, dtype=torch.float64)

            def brute_pin(q=q, k=k, v=v, causal=causal):
                o, lse = oracle.attention(q, k, v, causal, 0.3, lib=lib)
                bo, bl = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, 0.3)
                return _ok(o, bo) and _ok(lse, bl)
            pin("brute %s" % ((Hq, Hkv, N, Nk, d, causal),), brute_pin)

    def sdpa_pin():
        q = torch.randn(1, 9, 4, 16, generator=g, dtype=torch.float64)
        k = torch.randn(1, 9, 2, 16, generator=g, dtype=torch.float64)
        v = torch.randn(1, 9, 2, 16, generator=g, dtype=torch.float64)
        o, _ = oracle.attention(q, k, v, True, 0.25, lib=lib)
        ref = F.scaled_dot_product_attention(
            q.transpose(1, 2), k.transpose(1, 2).repeat_interleave(2, 1),
            v.transpose(1, 2).repeat_interleave(2, 1), is_causal=True, scale=0.25)
        return _ok(o, ref.transpose(1, 2).numpy())
    pin("sdpa", sdpa_pin)

    def decode_sdpa_pin():
        lens = [2, 5, 3]
        cu = torch.tensor([0, 2, 7, 10], dtype=torch.int32)
        q = torch.randn(3, 2, 8, generator=g, dtype=torch.float64)
        kc = torch.randn(10, 1, 8, generator=g, dtype=torch.float64)
        vc = torch.randn(10, 1, 8, generator=g, dtype=torch.float64)
        o, lse = oracle.decode(q, kc, vc, cu, 0.5, lib=lib)
        good = True
        for b in range(3):
            s, e = int(cu[b]), int(cu[b + 1])
            kh = kc[s:e].transpose(0, 1).expand(2, lens[b], 8)
            vh = vc[s:e].transpose(0, 1).expand(2, lens[b], 8)
            ref = F.scaled_dot_product_attention(q[b][:, None], kh, vh, scale=0.5)[:, 0]
            good &= _ok(o[b], ref.numpy())
            good &= _ok(lse[b], torch.logsumexp(0.5 * (kh @ q[b][:, :, None])[..., 0], -1).numpy())
        return good
    pin("decode sdpa", decode_sdpa_pin)
    return failures


def _build_variant(tmp_path, name, src_text):
    cpath = tmp_path / ("%s.c" % name)
    cpath.write_text(src_text)
    so = str(tmp_path / ("lib%s.so" % name))
    oracle.compile_source(str(cpath), so)
    return oracle.load_library(so)


def test_unmodified_oracle_passes_battery(tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert battery(_build_variant(tmp_path, "control", text)) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_battery_rejects_planted_mistake(tmp_path, mutant):
    old, new = MUTANTS[mutant]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation anchor not found: %r" % old
    name = "m" + str(abs(hash(mutant)) % 10**8)
    failures = battery(_build_variant(tmp_path, name, text.replace(old, new)))
    assert failures, "no pin caught the planted mistake %r" % mutant

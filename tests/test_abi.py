"""The C ABI of libfa.so without a GPU: every symbol include/fa.h declares is
exported, and argument errors are reported as status codes before anything is
enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from exact_io_aware_fa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
F32, BF16 = 0, 1


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("fa_fwd", "fa_fwd_varlen", "fa_decode", "fa_decode_workspace_bytes", "fa_decode_noalloc",
              "fa_decode_paged",
              "fa_decode_paged_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_str",
              "fa_last_error", "fa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(fa_lib):
    raw = ctypes.CDLL(binding.library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), "libfa.so does not export %s" % name


def test_abi_version_and_status_names(fa_lib):
    assert fa_lib.fa_abi_version() == 5
    names = [fa_lib.fa_status_str(s).decode() for s in range(5)]
    assert names == ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE",
                     "FA_ERR_HIP"]
    assert fa_lib.fa_status_str(99).decode() == "FA_ERR_UNKNOWN"


def _fwd(lib, dtype=BF16, q=None, k=None, v=None, o=None, lse=None, B=1, Hq=2, Hkv=1, N=4, Nk=4,
         d=64, causal=0, scale=0.125):
    return lib.fa_fwd(dtype, q, k, v, o, lse, B, Hq, Hkv, N, Nk, d, causal, scale, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=7), FA_ERR_INVALID_ARG),
    (dict(B=-1), FA_ERR_INVALID_ARG),
    (dict(N=-3), FA_ERR_INVALID_ARG),
    (dict(Nk=-1), FA_ERR_INVALID_ARG),
    (dict(Hq=0), FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), FA_ERR_INVALID_ARG),
    (dict(d=0), FA_ERR_INVALID_ARG),
    (dict(d=96), FA_ERR_UNSUPPORTED),
    (dict(d=256), FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), FA_ERR_INVALID_ARG),
    (dict(scale=0.0), FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), FA_ERR_INVALID_ARG),
    (dict(), FA_ERR_INVALID_ARG),                       # null pointers with work to do
    (dict(B=0), FA_OK),                                  # no work: nothing touched
    (dict(N=0), FA_OK),
])
def test_fwd_validation(fa_lib, kwargs, status):
    st = _fwd(fa_lib, **kwargs)
    assert st == status
    if status != FA_OK:
        assert fa_lib.fa_last_error().decode() != ""
    else:
        assert fa_lib.fa_last_error().decode() == ""


def _fwd_varlen(lib, dtype=BF16, ptr=None, cu=None, max_q=4, max_k=6, total_q=8, total_k=12, B=2, Hq=2,
                Hkv=1, d=64, causal=1, scale=0.125):
    return lib.fa_fwd_varlen(dtype, ptr, ptr, ptr, cu, cu, max_q, max_k, total_q, total_k, ptr, ptr, B, Hq, Hkv, d,
                             causal, scale, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=F32), FA_ERR_UNSUPPORTED),
    (dict(dtype=7), FA_ERR_INVALID_ARG),
    (dict(B=-1), FA_ERR_INVALID_ARG),
    (dict(max_q=-1), FA_ERR_INVALID_ARG),
    (dict(max_k=-1), FA_ERR_INVALID_ARG),
    (dict(total_q=-1), FA_ERR_INVALID_ARG),
    (dict(total_k=-1), FA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), FA_ERR_INVALID_ARG),
    (dict(d=96), FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), FA_ERR_INVALID_ARG),
    (dict(), FA_ERR_INVALID_ARG),                       # null pointers with work to do
    (dict(B=0), FA_OK),                                  # no work: nothing touched
    (dict(total_q=0), FA_OK),
    (dict(max_q=0), FA_OK),
])
def test_fwd_varlen_validation(fa_lib, kwargs, status):
    st = _fwd_varlen(fa_lib, **kwargs)
    assert st == status
    if status != FA_OK:
        assert fa_lib.fa_last_error().decode() != ""


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only check")
def test_fwd_varlen_alignment_and_aliasing_rejected(fa_lib):
    q, k, v, cu, o, lse = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000
    args = lambda q_, cu_, o_: fa_lib.fa_fwd_varlen(BF16, q_, k, v, cu_, cu_, 4, 6, 8, 12, o_, lse, 2, 2, 1, 64, 1,
                                                    0.125, None)
    assert args(q + 2, cu, o) == FA_ERR_INVALID_ARG and "aligned" in fa_lib.fa_last_error().decode()
    assert args(q, cu + 2, o) == FA_ERR_INVALID_ARG and "cu_seqlens" in fa_lib.fa_last_error().decode()
    assert args(q, cu, q) == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()


def _decode(lib, dtype=BF16, ptr=None, cu=None, max_len=100, B=2, Hq=8, Hkv=1, d=128,
            scale=0.1, ws=None, ws_bytes=0):
    return lib.fa_decode(dtype, ptr, ptr, ptr, cu, max_len, ptr, ptr, B, Hq, Hkv, d, scale, ws,
                         ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=F32), FA_ERR_UNSUPPORTED),
    (dict(dtype=5), FA_ERR_INVALID_ARG),
    (dict(B=-1), FA_ERR_INVALID_ARG),
    (dict(max_len=-1), FA_ERR_INVALID_ARG),
    (dict(Hq=8, Hkv=3), FA_ERR_INVALID_ARG),
    (dict(Hq=32, Hkv=1), FA_ERR_UNSUPPORTED),           # group of 32 query heads
    (dict(d=80), FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), FA_ERR_INVALID_ARG),
    (dict(), FA_ERR_INVALID_ARG),                        # null pointers
    (dict(B=0), FA_OK),
])
def test_decode_validation(fa_lib, kwargs, status):
    assert _decode(fa_lib, **kwargs) == status


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only check")
def test_misaligned_and_aliased_pointers_rejected(fa_lib):
    a, b2, c, o, lse = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    st = fa_lib.fa_fwd(BF16, a + 2, b2, c, o, lse, 1, 2, 1, 4, 4, 64, 0, 0.125, None)
    assert st == FA_ERR_INVALID_ARG and "aligned" in fa_lib.fa_last_error().decode()
    st = fa_lib.fa_fwd(BF16, a, b2, c, a, lse, 1, 2, 1, 4, 4, 64, 0, 0.125, None)   # o == q
    assert st == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only check")
def test_decode_workspace_checked(fa_lib):
    need = fa_lib.fa_decode_workspace_bytes(2, 8, 1, 128, 100)
    assert need > 0
    p, cu, ws = 0x100000, 0x200000, 0x300000
    st = _decode(fa_lib, ptr=p, cu=cu, ws=ws, ws_bytes=need - 1)
    assert st == FA_ERR_WORKSPACE
    st = _decode(fa_lib, ptr=p, cu=cu, ws=None, ws_bytes=need)
    assert st == FA_ERR_WORKSPACE


def test_workspace_size_query(fa_lib):
    f = fa_lib.fa_decode_workspace_bytes
    assert f(0, 64, 8, 128, 1000) == 0
    assert f(32, 64, 8, 128, 0) == 0
    small, large = f(32, 64, 8, 128, 512), f(32, 64, 8, 128, 32768)
    assert 0 < small <= large
    # partial outputs (fp32, d per slot) plus one fp32 LSE per slot
    assert large < 32 * 64 * 128 * 4 * 64


def test_binding_refuses_cpu_tensors(fa_lib):
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous(), False, 0.125)



# Caller-given outputs and mixed input dtypes are refused by the binding before
# any pointer reaches the library (an undersized or differently typed output
# would otherwise be written past its end).  CPU tensors suffice: these checks
# run before the device check.
def _bf(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_checks_fwd_outputs_and_dtypes(fa_lib):
    import torch
    q, k = _bf(1, 4, 2, 64), _bf(1, 4, 1, 64)
    with pytest.raises(ValueError, match="out must have shape"):
        binding.fwd(q, k, k, False, 0.125, out=_bf(1, 3, 2, 64))
    with pytest.raises(TypeError, match="out must be"):
        binding.fwd(q, k, k, False, 0.125, out=torch.zeros(1, 4, 2, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        binding.fwd(q, k, k, False, 0.125, lse=torch.zeros(1, 2, 3))
    with pytest.raises(TypeError, match="lse must be"):
        binding.fwd(q, k, k, False, 0.125, lse=torch.zeros(1, 2, 4, dtype=torch.float64))
    with pytest.raises(ValueError, match="contiguous"):
        binding.fwd(q, k, k, False, 0.125, out=_bf(1, 4, 64, 2).transpose(2, 3))
    with pytest.raises(TypeError, match="k must share"):
        binding.fwd(q, k.float(), k, False, 0.125)


def test_binding_checks_varlen_outputs(fa_lib):
    import torch
    q, k = _bf(6, 2, 64), _bf(9, 1, 64)
    cu = torch.tensor([0, 6], dtype=torch.int32)
    cuk = torch.tensor([0, 9], dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        binding.fwd_varlen(q, k, k, cu, cuk, 6, 9, True, 0.125, out=_bf(5, 2, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        binding.fwd_varlen(q, k, k, cu, cuk, 6, 9, True, 0.125, lse=torch.zeros(6, 2))
    with pytest.raises(TypeError, match="v must share"):
        binding.fwd_varlen(q, k, k.float(), cu, cuk, 6, 9, True, 0.125)


def test_binding_checks_decode_outputs_and_dtypes(fa_lib):
    import torch
    q, kc = _bf(2, 8, 128), _bf(40, 2, 128)
    cu = torch.tensor([0, 10, 40], dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        binding.decode(q, kc, kc, cu, 30, 0.1, out=_bf(1, 8, 128))
    with pytest.raises(TypeError, match="out must be"):
        binding.decode(q, kc, kc, cu, 30, 0.1, out=torch.zeros(2, 8, 128))
    with pytest.raises(ValueError, match="lse must have shape"):
        binding.decode(q, kc, kc, cu, 30, 0.1, lse=torch.zeros(2, 4))
    with pytest.raises(TypeError, match="k_cache must share"):
        binding.decode(q, kc.float(), kc, cu, 30, 0.1)


def test_binding_checks_decode_paged_outputs_and_dtypes(fa_lib):
    import torch
    q, pages, new = _bf(2, 8, 128), _bf(4, 64, 2, 128), _bf(2, 2, 128)
    table = torch.zeros(2, 2, dtype=torch.int32)
    lens = torch.tensor([10, 20], dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        binding.decode_paged(q, pages, pages, table, lens, 20, 0.1, new, new, out=_bf(2, 8, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        binding.decode_paged(q, pages, pages, table, lens, 20, 0.1, new, new, lse=torch.zeros(8))
    with pytest.raises(TypeError, match="k_new must share"):
        binding.decode_paged(q, pages, pages, table, lens, 20, 0.1, new.float(), new)
    with pytest.raises(TypeError, match="v_cache must share"):
        binding.decode_paged(q, pages, pages.float(), table, lens, 20, 0.1, new, new)


def test_binding_checks_bwd_outputs_and_dtypes(fa_lib):
    import torch
    q, k = _bf(1, 4, 2, 64), _bf(1, 5, 1, 64)
    lse = torch.zeros(1, 2, 4)
    with pytest.raises(TypeError, match="dout must share"):
        binding.bwd(q, k, k, q, lse, q.float(), True, 0.125)
    with pytest.raises(TypeError, match="o must share"):
        binding.bwd(q, k, k, q.float(), lse, q, True, 0.125)
    with pytest.raises(ValueError, match="dq must have shape"):
        binding.bwd(q, k, k, q, lse, q, True, 0.125, dq=_bf(1, 4, 2, 32))
    with pytest.raises(ValueError, match="dk must have shape"):
        binding.bwd(q, k, k, q, lse, q, True, 0.125, dk=_bf(1, 4, 1, 64))
    with pytest.raises(TypeError, match="dv must be"):
        binding.bwd(q, k, k, q, lse, q, True, 0.125, dv=torch.zeros(1, 5, 1, 64))


def _paged(lib, dtype=BF16, q=None, kn=None, vn=None, kc=None, vc=None, table=None, lens=None, num_blocks=8,
           block_size=64, max_blocks=4, max_len=200, o=None, lse=None, B=2, Hq=8, Hkv=2, d=128, scale=0.1, ws=None,
           ws_bytes=0):
    return lib.fa_decode_paged(dtype, q, kn, vn, kc, vc, table, lens, num_blocks, block_size, max_blocks, max_len,
                               o, lse, B, Hq, Hkv, d, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=F32), FA_ERR_UNSUPPORTED),
    (dict(dtype=4), FA_ERR_INVALID_ARG),
    (dict(B=-1), FA_ERR_INVALID_ARG),
    (dict(max_len=-1), FA_ERR_INVALID_ARG),
    (dict(num_blocks=-1), FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), FA_ERR_INVALID_ARG),
    (dict(Hq=64, Hkv=2), FA_ERR_UNSUPPORTED),           # group of 32 query heads
    (dict(d=32), FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), FA_ERR_INVALID_ARG),
    (dict(block_size=16), FA_ERR_INVALID_ARG),          # below one 32-key tile
    (dict(block_size=96), FA_ERR_INVALID_ARG),          # not a power of two
    (dict(kn=0x1000), FA_ERR_INVALID_ARG),              # k_new without v_new
    (dict(max_len=257), FA_ERR_INVALID_ARG),            # 4 blocks of 64 rows hold 256
    (dict(), FA_ERR_INVALID_ARG),                       # null pointers
    (dict(B=0), FA_OK),
])
def test_decode_paged_validation(fa_lib, kwargs, status):
    assert _paged(fa_lib, **kwargs) == status
    if status != FA_OK:
        assert fa_lib.fa_last_error().decode() != ""


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only check")
def test_decode_paged_capacity_alignment_aliasing_and_workspace(fa_lib):
    need = fa_lib.fa_decode_paged_workspace_bytes(2, 8, 2, 128, 200)
    assert need > fa_lib.fa_decode_workspace_bytes(2, 8, 2, 128, 201)
    q, kn, vn, kc, vc = 0x100000, 0x200000, 0x300000, 0x1000000, 0x2000000
    table, lens, o, lse, ws = 0x400000, 0x500000, 0x600000, 0x700000, 0x800000
    call = lambda **kw: _paged(fa_lib, **{**dict(q=q, kn=kn, vn=vn, kc=kc, vc=vc, table=table, lens=lens, o=o,
                                                 lse=lse, ws=ws, ws_bytes=need), **kw})
    # exactly full with the append: 4 blocks of 64 rows hold 255 cached rows + 1
    assert call(max_len=256) == FA_ERR_INVALID_ARG and "exceeds" in fa_lib.fa_last_error().decode()
    # without it 256 rows fit: the call gets past the capacity check to the workspace check
    assert call(max_len=256, kn=None, vn=None, ws_bytes=0) == FA_ERR_WORKSPACE
    assert call(table=table + 2) == FA_ERR_INVALID_ARG and "4-byte" in fa_lib.fa_last_error().decode()
    assert call(kn=kn + 8) == FA_ERR_INVALID_ARG and "aligned" in fa_lib.fa_last_error().decode()
    assert call(o=q) == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()
    assert call(ws=kc + 64) == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()
    assert call(vc=kc + 1024) == FA_ERR_INVALID_ARG                # the two written caches overlap
    assert call(ws_bytes=need - 1) == FA_ERR_WORKSPACE
    assert call(ws=None) == FA_ERR_WORKSPACE


def test_decode_paged_workspace_size_query(fa_lib):
    f = fa_lib.fa_decode_paged_workspace_bytes
    assert f(0, 64, 8, 128, 1000) == 0
    assert f(32, 64, 8, 128, 0) > 0                      # the appended row alone is work
    assert 0 < f(32, 64, 8, 128, 512) <= f(32, 64, 8, 128, 32768)


def _bwd(lib, dtype=BF16, p=None, B=1, Hq=4, Hkv=2, N=64, Nk=64, d=128, causal=1, scale=0.1, ws=None,
         ws_bytes=0):
    return lib.fa_bwd(dtype, p, p, p, p, p, p, p, p, p, B, Hq, Hkv, N, Nk, d, causal, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=F32), FA_ERR_UNSUPPORTED),
    (dict(dtype=9), FA_ERR_INVALID_ARG),
    (dict(B=-1), FA_ERR_INVALID_ARG),
    (dict(N=-1), FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), FA_ERR_INVALID_ARG),
    (dict(d=96), FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), FA_ERR_INVALID_ARG),
    (dict(), FA_ERR_INVALID_ARG),                       # null pointers
    (dict(B=0), FA_OK),
    (dict(N=0, Nk=0), FA_OK),
])
def test_bwd_validation(fa_lib, kwargs, status):
    assert _bwd(fa_lib, **kwargs) == status


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only check")
def test_bwd_alignment_aliasing_and_workspace(fa_lib):
    need = fa_lib.fa_bwd_workspace_bytes(1, 4, 64)
    assert need >= 2 * 4 * 64 * 4 and fa_lib.fa_bwd_workspace_bytes(1, 4, 0) == 0
    base = [0x100000 * (i + 1) for i in range(10)]
    q, k, v, o, lse, do, dq, dk, dv, ws = base
    call = lambda **kw: fa_lib.fa_bwd(BF16, *[kw.get(n, x) for n, x in zip(
        ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"), (q, k, v, o, lse, do, dq, dk, dv))],
        1, 4, 2, 64, 64, 128, 1, 0.1, kw.get("ws", ws), kw.get("ws_bytes", need), None)
    assert call(dq=dq + 4) == FA_ERR_INVALID_ARG and "aligned" in fa_lib.fa_last_error().decode()
    assert call(dq=q) == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()
    assert call(dk=dv) == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()
    assert call(ws=do) == FA_ERR_INVALID_ARG and "alias" in fa_lib.fa_last_error().decode()
    assert call(ws_bytes=need - 1) == FA_ERR_WORKSPACE



def test_decode_noalloc_refuses_before_touching_the_device(fa_lib):
    """fa_decode_noalloc checks its arguments like fa_decode, and refuses sizes
    whose partial results exceed the static array, before any device call."""
    call = lambda B, Hq, Hkv, L, d=128, o=0x100000: fa_lib.fa_decode_noalloc(
        BF16, 0x200000, 0x300000, 0x400000, 0x500000, L, o, 0x600000, B, Hq, Hkv, d, 0.1, None)
    assert call(1024, 16, 1, 1 << 22) == FA_ERR_WORKSPACE
    assert b"static array" in fa_lib.fa_last_error()
    assert call(4, 64, 1, 1000) == FA_ERR_UNSUPPORTED                 # group of 64 query heads
    assert call(4, 8, 2, 1000, d=96) == FA_ERR_UNSUPPORTED
    assert call(-1, 8, 2, 1000) == FA_ERR_INVALID_ARG
    assert call(4, 8, 2, 1000, o=0x200000) == FA_ERR_INVALID_ARG      # o aliases q
    assert call(0, 8, 2, 1000) == FA_OK                               # no work, no device call
    # the decode workload fits: 32 sequences, Hq 64, Hkv 8, d 128, caches up to 32768 rows
    assert binding.decode_workspace_bytes(32, 64, 8, 128, 32768) <= binding.DECODE_SCRATCH_BYTES

"""Exact, IO-aware attention forward for AMD MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fa.h``).  ``fwd`` and ``decode`` marshal torch tensors
to that ABI; they raise if the library is not built.  ``inputs`` holds the
seeded synthetic workloads.
"""
from .binding import (  # noqa: F401
    FA_BF16,
    FA_F32,
    FaError,
    abi_version,
    decode,
    decode_workspace_bytes,
    fwd,
    library_path,
    load_library,
)

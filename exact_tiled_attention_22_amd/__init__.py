"""Exact tiled attention (forward and backward) for AMD Instinct MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind the C ABI of ``include/fa.h``);
this package only loads it and marshals arguments.
"""

from .binding import (  # noqa: F401
    FA_BF16,
    FA_F16,
    FA_F32,
    FA_FP8_E4M3,
    FaError,
    abi_version,
    bwd,
    decode_workspace_bytes,
    fp8_prep,
    fwd,
    fwd_decode,
    last_error,
    lib,
    status_str,
)

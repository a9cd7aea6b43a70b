"""Exact tiled attention (forward, backward, decode, and the unfused comparison path) for AMD Instinct
MI355X (gfx950).

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
    DECODE_NOALLOC_BYTES,
    decode_workspace_bytes,
    fp8_prep,
    fp8_prep_qkv,
    fwd,
    fwd_decode,
    fwd_decode_noalloc,
    fwd_naive,
    fwd_rect,
    fwd_split,
    last_error,
    lib,
    naive_pv,
    naive_row_stride,
    naive_scores,
    naive_softmax,
    naive_workspace_bytes,
    split_workspace_bytes,
    status_str,
)

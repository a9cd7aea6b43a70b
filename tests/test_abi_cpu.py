"""The C ABI on a host without a GPU: the header is valid C99, the library loads and exports every
declared symbol, and argument validation returns the documented status before any HIP call.
No compute call is made here."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_tiled_attention_22_amd", "libfa.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_DTYPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_ARG = range(7)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_compiles_as_c99():
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "t.c")
        with open(src, "w") as f:
            f.write('#include "fa.h"\nint main(void) { fa_fp8_scales s = {0, 0, 0, 64}; '
                    'return (int)FA_OK + s.block * 0 + (int)sizeof(&fa_fwd) * 0; }\n')
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.dirname(HEADER),
                            src, "-c", "-o", os.path.join(td, "t.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_ex", "fa_fwd_rect", "fa_fwd_split", "fa_fwd_split_workspace_bytes",
                          "fa_bwd", "fa_fwd_decode", "fa_decode_workspace_bytes", "fa_fwd_decode_noalloc",
                          "fa_fp8_prep", "fa_status_str", "fa_last_error", "fa_abi_version",
                          "fa_naive_row_stride", "fa_naive_workspace_bytes", "fa_naive_scores",
                          "fa_naive_softmax", "fa_naive_pv", "fa_fwd_naive", "fa_fp8_prep_qkv"}
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, re.M), f"{n} not exported with C linkage"


def _fwd(lib, q=16, k=16, v=16, o=16, lse=None, B=1, H=1, N=8, d=128, causal=0, scale=0.1, dtype=2):
    f = lib.fa_fwd
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, vp] + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int, vp]
    return f(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


def test_validation_statuses(lib):
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.restype = ctypes.c_int
    assert lib.fa_abi_version() == 3
    big = 1 << 20  # fake, 16-aligned addresses: validation never dereferences them
    assert _fwd(lib, dtype=9) == FA_ERR_DTYPE
    assert _fwd(lib, N=-1) == FA_ERR_SHAPE
    assert _fwd(lib, causal=2) == FA_ERR_ARG
    assert _fwd(lib, scale=float("nan")) == FA_ERR_ARG
    assert _fwd(lib, scale=float("inf")) == FA_ERR_ARG
    assert _fwd(lib, d=96) == FA_ERR_UNSUPPORTED
    assert b"d=96" in lib.fa_last_error()
    assert _fwd(lib, N=0, q=None, k=None, v=None, o=None) == FA_OK  # empty problem: no-op
    assert _fwd(lib, B=0) == FA_OK
    assert _fwd(lib, q=None) == FA_ERR_NULL
    assert _fwd(lib, q=big + 8, k=big * 2, v=big * 3, o=big * 4) == FA_ERR_ALIGN
    assert _fwd(lib, q=big, k=big * 2, v=big * 3, o=big * 4, lse=big * 5 + 4) == FA_ERR_ALIGN
    assert _fwd(lib, q=big, k=big * 2, v=big * 3, o=big) == FA_ERR_ARG  # o aliases q
    assert _fwd(lib, B=1 << 16, H=1 << 16, q=big, k=big * 2, v=big * 3, o=big * 4) == FA_ERR_SHAPE
    far = 1 << 40  # disjoint fake regions for the longest sequences
    assert _fwd(lib, N=1 << 21, q=far, k=far * 2, v=far * 3, o=far * 4, lse=far * 5) == FA_ERR_SHAPE
    for s in range(8):
        assert lib.fa_status_str(s)
    assert lib.fa_status_str(99) == b"unknown fa_status"


def test_prep_validation_statuses(lib):
    f = lib.fa_fp8_prep
    vp = ctypes.c_void_p
    f.argtypes = [vp, ctypes.c_int, vp, vp, vp] + [ctypes.c_int] * 4 + [vp]
    f.restype = ctypes.c_int
    big = 1 << 20
    good = (ctypes.c_int8 * 128)(*([1, -1] * 64))
    bad = (ctypes.c_int8 * 128)(*([1] * 127 + [0]))
    assert f(big, 3, big * 2, big * 3, None, 64, 1, 64, 128, None) == FA_ERR_DTYPE
    assert f(big, 2, big * 2, big * 3, None, 0, 1, 64, 128, None) == FA_ERR_ARG
    assert f(big, 2, big * 2, big * 3, None, 64, 1, 64, 96, None) == FA_ERR_UNSUPPORTED
    assert f(big, 2, big * 2, big * 3, ctypes.cast(bad, vp), 64, 1, 64, 128, None) == FA_ERR_ARG
    assert f(big, 2, big * 2, big * 3, ctypes.cast(good, vp), 64, 0, 64, 128, None) == FA_OK
    assert f(None, 2, big * 2, big * 3, ctypes.cast(good, vp), 64, 1, 64, 128, None) == FA_ERR_NULL
    assert f(big + 4, 2, big * 2, big * 3, None, 64, 1, 64, 128, None) == FA_ERR_ALIGN


def test_prep_qkv_validation_statuses(lib):
    f = lib.fa_fp8_prep_qkv
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, ctypes.c_int] + [vp] * 7 + [ctypes.c_int] * 4 + [vp]
    f.restype = ctypes.c_int
    big = 1 << 36
    x = [big * (i + 1) for i in range(3)]         # q k v (fake, never touched)
    c8 = [big * (i + 4) for i in range(3)]        # q8 k8 v8
    sc = [big * (i + 7) for i in range(3)]        # scales
    good = (ctypes.c_int8 * 128)(*([1, -1] * 64))
    bad = (ctypes.c_int8 * 128)(*([1] * 127 + [0]))

    def call(xx=None, cc=None, ss=None, dtype=2, signs=good, block=64, BH=2, N=100, d=128):
        return f(*(xx or x), dtype, *(cc or c8), *(ss or sc), signs, block, BH, N, d, None)

    assert call(dtype=3) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(block=0) == FA_ERR_ARG
    assert call(signs=bad) == FA_ERR_ARG
    assert call(BH=-1) == FA_ERR_SHAPE
    assert call(cc=[c8[0], None, c8[2]]) == FA_ERR_NULL
    assert call(ss=[sc[0], sc[1], sc[2] + 4]) == FA_ERR_ALIGN
    assert call(cc=[c8[0], c8[0], c8[2]]) == FA_ERR_ARG  # q8 and k8 alias
    assert call(ss=[x[1], sc[1], sc[2]]) == FA_ERR_ARG    # a scale array inside k
    assert call(N=0) == FA_OK


def test_bwd_validation_statuses(lib):
    f = lib.fa_bwd
    vp = ctypes.c_void_p
    f.argtypes = [vp] * 10 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    big = 1 << 24  # fake, 16-aligned, disjoint 16 MiB regions: validation never dereferences them
    ptrs = [big * (i + 1) for i in range(10)]  # q k v o lse dout dq dk dv delta

    def call(p=None, B=1, H=2, N=64, d=128, causal=0, scale=0.1, dtype=2):
        return f(*(p or ptrs), B, H, N, d, causal, scale, dtype, None)

    # every call below fails validation (or is empty), so nothing is ever launched on these fake pointers
    assert call(dtype=0) == FA_ERR_UNSUPPORTED   # float32 backward is not built
    assert call(dtype=3) == FA_ERR_UNSUPPORTED   # nor fp8
    assert call(dtype=9) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(causal=3) == FA_ERR_ARG
    assert call(scale=float("nan")) == FA_ERR_ARG
    assert call(N=-2) == FA_ERR_SHAPE
    assert call(N=0, p=[None] * 10) == FA_OK      # empty problem: no-op
    assert call(p=ptrs[:9] + [None]) == FA_ERR_NULL
    assert call(p=ptrs[:4] + [big * 5 + 4] + ptrs[5:]) == FA_ERR_ALIGN
    alias = list(ptrs)
    alias[6] = ptrs[0]  # dq aliases q
    assert call(p=alias) == FA_ERR_ARG
    alias = list(ptrs)
    alias[7] = ptrs[8]  # dk aliases dv
    assert call(p=alias) == FA_ERR_ARG


def test_decode_validation_statuses(lib):
    f = lib.fa_fwd_decode
    vp = ctypes.c_void_p
    f.argtypes = [vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp]
    f.restype = ctypes.c_int
    ws = lib.fa_decode_workspace_bytes
    ws.argtypes = [ctypes.c_int] * 5
    ws.restype = ctypes.c_size_t
    need = ws(2, 4, 1, 1000, 128)
    assert need > 0 and need % 16 == 0
    assert ws(0, 4, 1, 1000, 128) == 0
    big = 1 << 26
    p = [big * (i + 1) for i in range(5)]  # q k v o lse
    w = big * 7

    def call(pp=None, B=2, H=4, Nq=1, Nk=1000, d=128, causal=0, scale=0.1, dtype=2, work=w, nbytes=None):
        return f(*(pp or p), B, H, Nq, Nk, d, causal, scale, dtype, work, need if nbytes is None else nbytes, None)

    # every call below fails validation (or is empty): nothing is launched on these fake pointers
    assert call(dtype=0) == FA_ERR_UNSUPPORTED
    assert call(dtype=7) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(Nq=33, Nk=1000) == FA_ERR_UNSUPPORTED
    assert call(Nq=5, Nk=4) == FA_ERR_SHAPE
    assert call(causal=2) == FA_ERR_ARG
    assert call(scale=float("inf")) == FA_ERR_ARG
    assert call(nbytes=need - 1) == FA_ERR_ARG
    assert call(work=None) == FA_ERR_NULL
    assert call(work=w + 8) == FA_ERR_ALIGN
    assert call(work=p[1]) == FA_ERR_ARG  # workspace overlaps k
    assert call(pp=[p[0], p[1], p[2], p[0], p[4]]) == FA_ERR_ARG  # o aliases q
    assert call(Nq=0) == FA_OK


def test_decode_noalloc_validation_statuses(lib):
    f = lib.fa_fwd_decode_noalloc
    vp = ctypes.c_void_p
    f.argtypes = [vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int, vp]
    f.restype = ctypes.c_int
    ws = lib.fa_decode_workspace_bytes
    ws.argtypes = [ctypes.c_int] * 5
    ws.restype = ctypes.c_size_t
    limit = 64 << 20  # FA_DECODE_NOALLOC_BYTES
    big = 1 << 36
    p = [big * (i + 1) for i in range(5)]  # q k v o lse (fake, never touched)

    def call(pp=None, B=2, H=4, Nq=1, Nk=1000, d=128, causal=0, scale=0.1, dtype=2):
        return f(*(pp or p), B, H, Nq, Nk, d, causal, scale, dtype, None)

    # every call below fails validation (or is empty): nothing is launched, no device is touched
    assert call(dtype=0) == FA_ERR_UNSUPPORTED
    assert call(dtype=7) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(Nq=33) == FA_ERR_UNSUPPORTED
    assert call(Nq=5, Nk=4) == FA_ERR_SHAPE
    assert call(causal=2) == FA_ERR_ARG
    assert call(scale=float("nan")) == FA_ERR_ARG
    assert call(pp=[p[0], p[1], None, p[3], p[4]]) == FA_ERR_NULL
    assert call(pp=[p[0] + 4, p[1], p[2], p[3], p[4]]) == FA_ERR_ALIGN
    assert call(pp=[p[0], p[1], p[2], p[0], p[4]]) == FA_ERR_ARG  # o aliases q
    assert call(Nq=0) == FA_OK and call(B=0) == FA_OK
    # a shape whose workspace exceeds the library-held array is refused with a clear message
    B, H, Nq, Nk, d = 64, 64, 32, 4096, 256
    assert ws(B, H, Nq, Nk, d) > limit
    assert f(*p, B, H, Nq, Nk, d, 0, 0.1, 2, None) == FA_ERR_UNSUPPORTED
    lib.fa_last_error.restype = ctypes.c_char_p
    assert b"library-held" in lib.fa_last_error()


def test_rect_validation_statuses(lib):
    f = lib.fa_fwd_rect
    vp, ci = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp] * 5 + [ci] * 7 + [ctypes.c_float, ci, vp]
    f.restype = ci
    big = 1 << 26
    p = [big * (i + 1) for i in range(5)]  # q k v o lse

    def call(pp=None, B=2, H=4, Nq=100, Nk=300, q_start=0, d=128, causal=0, scale=0.1, dtype=2):
        return f(*(pp or p), B, H, Nq, Nk, q_start, d, causal, scale, dtype, None)

    # every call below fails validation (or is empty): nothing is launched on these fake pointers
    assert call(dtype=0) == FA_ERR_UNSUPPORTED  # float32: square fa_fwd only
    assert call(dtype=3) == FA_ERR_UNSUPPORTED
    assert call(dtype=9) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(Nq=-1) == FA_ERR_SHAPE
    assert call(Nk=-1) == FA_ERR_SHAPE
    assert call(causal=2) == FA_ERR_ARG
    assert call(scale=float("nan")) == FA_ERR_ARG
    assert call(q_start=5) == FA_ERR_ARG  # non-causal takes q_start 0
    assert call(causal=1, q_start=-1) == FA_ERR_ARG
    assert call(causal=1, q_start=201) == FA_ERR_ARG  # q_start + Nq > Nk
    assert call(causal=1, Nq=301, Nk=300) == FA_ERR_ARG
    assert call(Nk=0) == FA_ERR_SHAPE  # queries against no keys
    assert call(pp=[None] * 5) == FA_ERR_NULL
    assert call(pp=[p[0] + 8] + p[1:]) == FA_ERR_ALIGN
    assert call(pp=[p[0], p[1], p[2], p[1], p[4]]) == FA_ERR_ARG  # o aliases k
    assert call(pp=[p[0], p[1], p[2], p[3], p[3]]) == FA_ERR_ARG  # lse aliases o
    assert call(Nq=0, pp=[None] * 5) == FA_OK
    assert call(B=0, pp=[None] * 5) == FA_OK


def test_split_validation_statuses(lib):
    f = lib.fa_fwd_split
    vp, ci = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp] * 5 + [ci] * 7 + [ctypes.c_float, ci, ci, vp, ctypes.c_size_t, vp]
    f.restype = ci
    lib.fa_fwd_split_workspace_bytes.argtypes = [ci] * 5
    lib.fa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    wsb = lib.fa_fwd_split_workspace_bytes
    assert wsb(2, 4, 100, 128, 3) == 2 * 4 * 3 * 100 * 129 * 4
    assert wsb(0, 4, 100, 128, 3) == 0 and wsb(2, 4, 100, 128, 0) == 0
    big = 1 << 26
    p = [big * (i + 1) for i in range(6)]  # q k v o lse workspace
    need = wsb(2, 4, 100, 128, 4)

    def call(pp=None, B=2, H=4, Nq=100, Nk=300, q_start=0, d=128, causal=0, scale=0.1, dtype=2, ns=4, nb=need):
        q, k, v, o, lse, ws = pp or p
        return f(q, k, v, o, lse, B, H, Nq, Nk, q_start, d, causal, scale, dtype, ns, ws, nb, None)

    # every call below fails validation (or is empty): nothing is launched on these fake pointers
    assert call(dtype=0) == FA_ERR_UNSUPPORTED
    assert call(dtype=9) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(Nq=-1) == FA_ERR_SHAPE
    assert call(causal=2) == FA_ERR_ARG
    assert call(scale=float("inf")) == FA_ERR_ARG
    assert call(q_start=5) == FA_ERR_ARG
    assert call(causal=1, q_start=201) == FA_ERR_ARG
    assert call(ns=0) == FA_ERR_ARG and call(ns=65) == FA_ERR_ARG
    assert call(nb=need - 1) == FA_ERR_ARG  # workspace too small
    assert call(Nk=0) == FA_ERR_SHAPE
    assert call(pp=[p[0], p[1], p[2], p[3], p[4], None]) == FA_ERR_NULL
    assert call(pp=p[:5] + [p[5] + 8]) == FA_ERR_ALIGN
    assert call(pp=p[:5] + [p[3]]) == FA_ERR_ARG  # workspace aliases o
    assert call(pp=[p[0], p[1], p[2], p[0], p[4], p[5]]) == FA_ERR_ARG  # o aliases q
    assert call(Nq=0, pp=[None] * 6) == FA_OK


def test_naive_validation_statuses(lib):
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.fa_naive_row_stride.argtypes = [ci]
    lib.fa_naive_row_stride.restype = ci
    lib.fa_naive_workspace_bytes.argtypes = [ci] * 3
    lib.fa_naive_workspace_bytes.restype = ctypes.c_size_t
    assert [lib.fa_naive_row_stride(n) for n in (1, 63, 64, 65, 1000)] == [64, 64, 64, 128, 1024]
    assert lib.fa_naive_workspace_bytes(2, 3, 100) == 2 * 3 * 100 * 128 * 6
    assert lib.fa_naive_workspace_bytes(0, 3, 100) == 0
    f = lib.fa_fwd_naive
    f.argtypes = [vp] * 5 + [ci] * 5 + [ctypes.c_float, ci, vp, ctypes.c_size_t, vp]
    f.restype = ci
    need = lib.fa_naive_workspace_bytes(2, 4, 100)
    big = 1 << 26
    p = [big * (i + 1) for i in range(5)]  # q k v o lse
    w = big * 8

    def call(pp=None, B=2, H=4, N=100, d=128, causal=0, scale=0.1, dtype=2, work=w, nbytes=None):
        return f(*(pp or p), B, H, N, d, causal, scale, dtype, work, need if nbytes is None else nbytes, None)

    # every call below fails validation (or is empty): nothing is launched on these fake pointers
    assert call(dtype=0) == FA_ERR_UNSUPPORTED
    assert call(dtype=3) == FA_ERR_UNSUPPORTED
    assert call(dtype=9) == FA_ERR_DTYPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(N=-1) == FA_ERR_SHAPE
    assert call(causal=3) == FA_ERR_ARG
    assert call(scale=float("nan")) == FA_ERR_ARG
    assert call(nbytes=need - 1) == FA_ERR_ARG
    assert call(work=None) == FA_ERR_NULL
    assert call(work=w + 4) == FA_ERR_ALIGN
    assert call(work=p[2]) == FA_ERR_ARG  # workspace overlaps v
    assert call(pp=[p[0], p[1], p[2], p[2], p[4]]) == FA_ERR_ARG  # o aliases v
    assert call(N=0) == FA_OK
    sc = lib.fa_naive_scores
    sc.argtypes = [vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, ci, vp]
    sc.restype = ci
    assert sc(p[0], p[1], p[0], 2, 4, 100, 128, 0.1, 2, None) == FA_ERR_ARG  # s overlaps q
    assert sc(p[0], None, w, 2, 4, 100, 128, 0.1, 2, None) == FA_ERR_NULL
    sm = lib.fa_naive_softmax
    sm.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp]
    sm.restype = ci
    assert sm(w, w + 64, None, 2, 4, 100, 0, 2, None) == FA_ERR_ARG  # p overlaps s
    assert sm(w, p[0], None, 2, 4, 100, 2, 2, None) == FA_ERR_ARG  # causal = 2
    pv = lib.fa_naive_pv
    pv.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp]
    pv.restype = ci
    assert pv(w, p[2], p[2], 2, 4, 100, 128, 2, None) == FA_ERR_ARG  # o aliases v
    assert pv(w, p[2], p[3], 2, 4, 100, 64 + 1, 2, None) == FA_ERR_UNSUPPORTED

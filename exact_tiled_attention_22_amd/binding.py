"""Python binding of libfa.so (ctypes).  Argument marshalling only: every step of the attention
passes (forward, fp8 preparation, backward, decode, unfused path) runs in the library's HIP kernels.  torch supplies device memory
and the current stream.  There is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

ABI_VERSION = 3  # FA_ABI_VERSION of include/fa.h that these argument lists follow
FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {
    torch.float32: FA_F32,
    torch.float16: FA_F16,
    torch.bfloat16: FA_BF16,
    torch.float8_e4m3fn: FA_FP8_E4M3,
}

_lib = None


class FaError(RuntimeError):
    """Non-FA_OK status from the library; ``status`` holds the code."""

    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} -> {status_str(status)} ({detail})")
        self.status = status


class _Fp8Scales(ctypes.Structure):
    _fields_ = [
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block", ctypes.c_int),
    ]


def lib() -> ctypes.CDLL:
    """Load libfa.so from this package directory (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(or python -m exact_tiled_attention_22_amd.build_lib)")
    L = ctypes.CDLL(LIB_PATH)
    L.fa_abi_version.argtypes = []
    L.fa_abi_version.restype = ctypes.c_int
    if L.fa_abi_version() != ABI_VERSION:  # argument lists below follow this version of include/fa.h
        raise RuntimeError(f"{LIB_PATH} implements ABI version {L.fa_abi_version()}, this binding version "
                           f"{ABI_VERSION}: rebuild it with __graft_entry__.build()")
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.fa_fwd.restype = i
    L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, ctypes.POINTER(_Fp8Scales), vp]
    L.fa_fwd_ex.restype = i
    L.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, vp]
    L.fa_bwd.restype = i
    L.fa_fwd_rect.argtypes = [vp] * 5 + [i] * 7 + [f, i, vp]
    L.fa_fwd_rect.restype = i
    L.fa_fwd_split.argtypes = [vp] * 5 + [i] * 7 + [f, i, i, vp, ctypes.c_size_t, vp]
    L.fa_fwd_split.restype = i
    L.fa_fwd_split_workspace_bytes.argtypes = [i] * 5
    L.fa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    L.fa_fwd_decode.argtypes = [vp] * 5 + [i] * 6 + [f, i, vp, ctypes.c_size_t, vp]
    L.fa_fwd_decode.restype = i
    L.fa_fwd_decode_noalloc.argtypes = [vp] * 5 + [i] * 6 + [f, i, vp]
    L.fa_fwd_decode_noalloc.restype = i
    L.fa_decode_workspace_bytes.argtypes = [i] * 5
    L.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.fa_naive_row_stride.argtypes = [i]
    L.fa_naive_row_stride.restype = i
    L.fa_naive_workspace_bytes.argtypes = [i, i, i]
    L.fa_naive_workspace_bytes.restype = ctypes.c_size_t
    L.fa_naive_scores.argtypes = [vp, vp, vp, i, i, i, i, f, i, vp]
    L.fa_naive_scores.restype = i
    L.fa_naive_softmax.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.fa_naive_softmax.restype = i
    L.fa_naive_pv.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.fa_naive_pv.restype = i
    L.fa_fwd_naive.argtypes = [vp] * 5 + [i] * 5 + [f, i, vp, ctypes.c_size_t, vp]
    L.fa_fwd_naive.restype = i
    L.fa_fp8_prep.argtypes = [vp, i, vp, vp, vp, i, i, i, i, vp]
    L.fa_fp8_prep.restype = i
    L.fa_fp8_prep_qkv.argtypes = [vp, vp, vp, i] + [vp] * 7 + [i, i, i, i, vp]
    L.fa_fp8_prep_qkv.restype = i
    L.fa_status_str.argtypes = [i]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def last_error() -> str:
    return lib().fa_last_error().decode()


def abi_version() -> int:
    return int(lib().fa_abi_version())


def _check(status: int, func: str) -> None:
    if status != 0:
        raise FaError(status, func, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _out(t, shape, dtype, device, name):
    """A caller-supplied output must have exactly the size the kernels write (the C ABI takes bare
    pointers and cannot check it); None allocates one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _workspace(ws, need, device):
    """A uint8 device workspace of at least ``need`` bytes (allocated when None)."""
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return ws  # the library checks the size against the bytes it needs


def _check_qkv(q, k, v):
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported or mixed dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
        return_lse: bool = True, fp8_scales=None, block: int = 64):
    """Attention forward through fa_fwd_ex.  Returns (o, lse) (lse None if return_lse is False).

    fp8 inputs (torch.float8_e4m3fn codes) take ``fp8_scales = (sq, sk, sv)`` float32 tensors of
    shape [B, H, ceil(N / block)] (or None for unit scales) and produce a bfloat16 output.
    """
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = DTYPE_CODE[q.dtype]
    out_dtype = torch.bfloat16 if code == FA_FP8_E4M3 else q.dtype
    out = _out(out, q.shape, out_dtype, q.device, "out")
    if return_lse:
        lse = _out(lse, (B, H, N), torch.float32, q.device, "lse")
    s8 = None
    if fp8_scales is not None:
        if code != FA_FP8_E4M3:
            raise ValueError(f"fp8_scales apply to float8_e4m3fn inputs only, got {q.dtype}")
        if int(block) <= 0:
            raise ValueError(f"block must be positive, got {block}")
        if len(fp8_scales) != 3:
            raise ValueError("fp8_scales must be a triple (sq, sk, sv)")
        # the C ABI reads B*H*ceil(N/block) floats from each pointer: the tensors must hold exactly that
        shape = (B, H, -(-N // int(block)))
        for name, t in zip(("sq", "sk", "sv"), fp8_scales):
            if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != q.device
                    or tuple(t.shape) != shape or not t.is_contiguous()):
                desc = f"{t.dtype} {tuple(t.shape)} on {t.device}" if isinstance(t, torch.Tensor) else type(t).__name__
                raise ValueError(f"fp8 scale {name} must be a contiguous float32 tensor of shape {shape} on "
                                 f"{q.device}, got {desc}")
        sq, sk, sv = fp8_scales
        s8 = ctypes.pointer(_Fp8Scales(sq.data_ptr(), sk.data_ptr(), sv.data_ptr(), int(block)))
    st = lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse if return_lse else None),
                         B, H, N, d, int(bool(causal)), float(scale), code, s8, _stream(q.device))
    _check(st, "fa_fwd_ex")
    return out, (lse if return_lse else None)


def fwd_rect(q, k, v, *, causal: bool = False, q_start: int | None = None, scale: float | None = None, out=None,
             lse=None):
    """Attention of q [B, H, Nq, d] against k, v [B, H, Nk, d] through fa_fwd_rect.  Causal: query i
    sits at position q_start + i of the key sequence (default Nk - Nq, the last Nq positions); non-causal
    takes q_start 0.  Returns (o, lse)."""
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, H, Nk, d] of q's dtype")
    if q_start is None:
        q_start = Nk - Nq if causal else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out(out, q.shape, q.dtype, q.device, "out")
    lse = _out(lse, (B, H, Nq), torch.float32, q.device, "lse")
    st = lib().fa_fwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, int(q_start), d,
                           int(bool(causal)), float(scale), DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "fa_fwd_rect")
    return out, lse


def split_workspace_bytes(B: int, H: int, Nq: int, d: int, nsplit: int) -> int:
    return int(lib().fa_fwd_split_workspace_bytes(B, H, Nq, d, nsplit))


def fwd_split(q, k, v, *, nsplit: int, causal: bool = False, q_start: int | None = None, scale: float | None = None,
              out=None, lse=None, workspace=None):
    """fwd_rect with each query tile's keys split into `nsplit` shares merged afterwards (fa_fwd_split).
    `workspace`: a uint8 GPU tensor of at least split_workspace_bytes(...) bytes (allocated here if None).
    Returns (o, lse)."""
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, H, Nk, d] of q's dtype")
    if q_start is None:
        q_start = Nk - Nq if causal else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out(out, q.shape, q.dtype, q.device, "out")
    lse = _out(lse, (B, H, Nq), torch.float32, q.device, "lse")
    need = split_workspace_bytes(B, H, Nq, d, nsplit) if nsplit >= 1 else 0
    ws = _workspace(workspace, need, q.device)
    st = lib().fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, int(q_start), d,
                            int(bool(causal)), float(scale), DTYPE_CODE[q.dtype], int(nsplit), _ptr(ws),
                            ws.numel() if ws is not None else 0, _stream(q.device))
    _check(st, "fa_fwd_split")
    return out, lse


def decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(lib().fa_decode_workspace_bytes(B, H, Nq, Nk, d))


def fwd_decode(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None, workspace=None):
    """Decode-shape attention through fa_fwd_decode: q [B, H, Nq, d] (Nq <= 32, the last Nq positions)
    against k, v [B, H, Nk, d].  Returns (o, lse).  ``workspace`` is a uint8 device tensor of at least
    decode_workspace_bytes(...) bytes (allocated when not given)."""
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, H, Nk, d] of q's dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out(out, q.shape, q.dtype, q.device, "out")
    lse = _out(lse, (B, H, Nq), torch.float32, q.device, "lse")
    need = decode_workspace_bytes(B, H, Nq, Nk, d)
    workspace = _workspace(workspace, need, q.device)
    st = lib().fa_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, int(bool(causal)),
                             float(scale), DTYPE_CODE[q.dtype], _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(st, "fa_fwd_decode")
    return out, lse


DECODE_NOALLOC_BYTES = 64 << 20  # FA_DECODE_NOALLOC_BYTES: the library-held decode workspace per GPU


def fwd_decode_noalloc(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """fwd_decode without a workspace, through fa_fwd_decode_noalloc: the partial results go to the
    library's own device array (64 MiB per GPU), so the call allocates nothing when ``out`` and ``lse`` are
    given.  Calls overlapping in time on one GPU race on that array.  Returns (o, lse)."""
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, H, Nk, d] of q's dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out(out, q.shape, q.dtype, q.device, "out")
    lse = _out(lse, (B, H, Nq), torch.float32, q.device, "lse")
    st = lib().fa_fwd_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d,
                                     int(bool(causal)), float(scale), DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "fa_fwd_decode_noalloc")
    return out, lse


def naive_row_stride(N: int) -> int:
    """Row stride (elements) of the unfused path's score and probability matrices: N rounded up to 64."""
    return int(lib().fa_naive_row_stride(N))


def naive_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(lib().fa_naive_workspace_bytes(B, H, N))


def naive_scores(q, k, *, scale: float | None = None, s=None):
    """Unfused step 1 through fa_naive_scores: s = scale q k^T as float32 [B, H, N, ld]."""
    _check_qkv(q, k, k)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = _out(s, (B, H, N, naive_row_stride(N)), torch.float32, q.device, "s")
    st = lib().fa_naive_scores(_ptr(q), _ptr(k), _ptr(s), B, H, N, d, float(scale), DTYPE_CODE[q.dtype],
                               _stream(q.device))
    _check(st, "fa_naive_scores")
    return s


def naive_softmax(s, *, dtype, causal: bool = False, p=None, lse=None):
    """Unfused step 2 through fa_naive_softmax: p = softmax(s [+ causal mask]) of ``dtype``
    [B, H, N, ld] (zero beyond column N) and lse [B, H, N]."""
    if not s.is_cuda or s.dtype != torch.float32 or s.dim() != 4 or not s.is_contiguous():
        raise ValueError("s must be a contiguous float32 [B, H, N, ld] GPU tensor")
    B, H, N, ld = s.shape
    if ld != naive_row_stride(N):
        raise ValueError(f"s rows must be {naive_row_stride(N)} elements apart, got {ld}")
    p = _out(p, s.shape, dtype, s.device, "p")
    lse = _out(lse, (B, H, N), torch.float32, s.device, "lse")
    st = lib().fa_naive_softmax(_ptr(s), _ptr(p), _ptr(lse), B, H, N, int(bool(causal)), DTYPE_CODE[dtype],
                                _stream(s.device))
    _check(st, "fa_naive_softmax")
    return p, lse


def naive_pv(p, v, *, out=None):
    """Unfused step 3 through fa_naive_pv: o = p v, [B, H, N, d] of v's dtype."""
    if not (p.is_cuda and v.is_cuda and p.is_contiguous() and v.is_contiguous()) or v.dim() != 4:
        raise ValueError("p and v must be contiguous 4-D GPU tensors")
    B, H, N, d = v.shape
    if p.shape != (B, H, N, naive_row_stride(N)) or p.dtype != v.dtype:
        raise ValueError("p must be [B, H, N, ld] of v's dtype")
    out = _out(out, v.shape, v.dtype, v.device, "out")
    st = lib().fa_naive_pv(_ptr(p), _ptr(v), _ptr(out), B, H, N, d, DTYPE_CODE[v.dtype], _stream(v.device))
    _check(st, "fa_naive_pv")
    return out


def fwd_naive(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None, workspace=None):
    """Unfused attention through fa_fwd_naive (the three steps, s and p in ``workspace``, a uint8 device
    tensor of at least naive_workspace_bytes(B, H, N) bytes, allocated when not given).  Returns (o, lse)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out(out, q.shape, q.dtype, q.device, "out")
    lse = _out(lse, (B, H, N), torch.float32, q.device, "lse")
    workspace = _workspace(workspace, naive_workspace_bytes(B, H, N), q.device)
    st = lib().fa_fwd_naive(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, int(bool(causal)),
                            float(scale), DTYPE_CODE[q.dtype], _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(st, "fa_fwd_naive")
    return out, lse


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
        delta=None):
    """Attention backward through fa_bwd: gradients (dq, dk, dv) of fwd's output for the output
    gradient ``dout``; ``o`` and ``lse`` are fwd's results for the same call.  float16/bfloat16, d in
    {64, 128, 256}.  ``delta`` is the float32 [B, H, N] workspace (allocated when not given)."""
    _check_qkv(q, k, v)
    for t in (o, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError("o and dout must match q in shape, dtype and device, contiguous")
    B, H, N, d = q.shape
    if (lse is None or lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 [B, H, N] tensor on {q.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _out(dq, q.shape, q.dtype, q.device, "dq")
    dk = _out(dk, q.shape, q.dtype, q.device, "dk")
    dv = _out(dv, q.shape, q.dtype, q.device, "dv")
    delta = _out(delta, (B, H, N), torch.float32, q.device, "delta")
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      _ptr(delta), B, H, N, d, int(bool(causal)), float(scale), DTYPE_CODE[q.dtype],
                      _stream(q.device))
    _check(st, "fa_bwd")
    return dq, dk, dv


def _sign_buffer(signs, d: int):
    """The rotation signs as the host int8 array fa_fp8_prep reads: exactly d values, each +1 or -1."""
    sign_list = [int(s) for s in (signs.tolist() if hasattr(signs, "tolist") else signs)]
    if len(sign_list) != d:
        raise ValueError(f"signs must hold d = {d} values, got {len(sign_list)}")
    if any(s not in (1, -1) for s in sign_list):
        raise ValueError("signs must be +1 or -1")
    return (ctypes.c_int8 * d)(*sign_list)


def fp8_prep(x, signs=None, block: int = 64, out=None, scales=None):
    """Block absmax e4m3 quantisation of x [B, H, N, d] (or [BH, N, d]) through fa_fp8_prep.

    signs: None or a length-d sequence of +1/-1 (host values) for the Hadamard rotation.
    Returns (codes as torch.float8_e4m3fn, scales float32 [..., ceil(N / block)]).
    """
    if not x.is_cuda or not x.is_contiguous() or x.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError("x must be a contiguous float32/float16/bfloat16 GPU tensor")
    if x.dim() < 3:
        raise ValueError("x must be [..., N, d]")
    N, d = x.shape[-2], x.shape[-1]
    BH = x.numel() // max(1, N * d) if N * d else int(math.prod(x.shape[:-2]))
    nblk = -(-N // block) if block > 0 else 0
    out = _out(out, x.shape, torch.float8_e4m3fn, x.device, "out")
    scales = _out(scales, tuple(x.shape[:-2]) + (max(nblk, 0),), torch.float32, x.device, "scales")
    sign_buf = None if signs is None else _sign_buffer(signs, d)
    st = lib().fa_fp8_prep(_ptr(x), DTYPE_CODE[x.dtype], _ptr(out), _ptr(scales),
                           ctypes.cast(sign_buf, ctypes.c_void_p) if sign_buf is not None else None,
                           int(block), int(BH), int(N), int(d), _stream(x.device))
    _check(st, "fa_fp8_prep")
    return out, scales


def fp8_prep_qkv(q, k, v, signs=None, block: int = 64):
    """fp8_prep of q, k (rotated with ``signs``, if given) and v (never rotated) in one launch
    (fa_fp8_prep_qkv).  Returns ((q8, sq), (k8, sk), (v8, sv)), bitwise what three fp8_prep calls give."""
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.float32, torch.float16, torch.bfloat16):
            raise ValueError("q, k, v must be contiguous float32/float16/bfloat16 GPU tensors")
    if q.dim() < 3 or q.shape != k.shape or q.shape != v.shape or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one [..., N, d] shape and dtype")
    N, d = q.shape[-2], q.shape[-1]
    BH = int(math.prod(q.shape[:-2]))
    nblk = -(-N // block) if block > 0 else 0
    outs = [(torch.empty(q.shape, dtype=torch.float8_e4m3fn, device=q.device),
             torch.empty(tuple(q.shape[:-2]) + (max(nblk, 0),), dtype=torch.float32, device=q.device)) for _ in range(3)]
    sign_buf = None if signs is None else _sign_buffer(signs, d)
    st = lib().fa_fp8_prep_qkv(_ptr(q), _ptr(k), _ptr(v), DTYPE_CODE[q.dtype], *(_ptr(o[0]) for o in outs),
                               *(_ptr(o[1]) for o in outs),
                               ctypes.cast(sign_buf, ctypes.c_void_p) if sign_buf is not None else None,
                               int(block), BH, int(N), int(d), _stream(q.device))
    _check(st, "fa_fp8_prep_qkv")
    return tuple(outs)

"""FP8 path of the oracle: e4m3 codec, Walsh-Hadamard rotation, block absmax quantisation
(test infrastructure only).

The pages name the ingredients but no numbers (FlashAttention-3 article, "Drei technische Hebel",
item 3 "FP8-Blockquantisierung": matrices are handled block by block in eight bits and a Hadamard
transform reduces the quantisation error; "Praxischeck", "Präzision": same; concept card
"FlashAttention 2 + 3 — speicherbewusste Attention-Kernels", "Kernpunkte": FP8 with absmax
scaling).  The readings used here, all of which the GPU path follows too:

* format: OCP e4m3fn (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, only
  S.1111.111 is NaN, largest finite 448, subnormal step 2^-9); conversion is round-to-nearest-even,
  magnitudes >= 464 saturate to 448 (never reached by the quantiser below);
* rotation: x' = (x * s) H_d / sqrt(d) applied to every row of Q and K with one shared random sign
  vector s, H_d the Sylvester Hadamard matrix; because (D_s H_d / sqrt(d)) is orthogonal,
  Q' K'^T = Q K^T exactly in real arithmetic.  V is not rotated;
* block: one scale per ``block`` consecutive rows of one (batch, head) over all d columns; the last
  block may be partial;
* absmax: amax = max |x'| over the block, scale = amax / 448, code = e4m3(x' * (448 / amax));
  an all-zero block gets scale 1 and zero codes.  The dequantised value is code * scale.

Because the quantiser turns floating point into integer codes, the oracle takes those decisions in
the same float32 precision and order as the kernel: float32 sign flip, float32 butterflies with
strides 1, 2, 4, ..., d/2 (each stage maps a pair (a, b) to (a + b, a - b)), a float32 multiply by
the float32 value of 1/sqrt(d), a float32 division 448/amax, a float32 multiply, then the e4m3
rounding.  Everything downstream of the codes (dequantisation, attention) is float64.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_ref

E4M3_MAX = 448.0
_E4M3_NAN = 0x7F
_F32_MAX = np.float32(np.finfo(np.float32).max)


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    norm = (8.0 + m) * np.exp2(e.astype(np.float64) - 10.0)
    mag = np.where(e == 0, sub, norm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """float32/float64 values -> uint8 e4m3fn codes, round-to-nearest-even, saturating at 448.

    The sign bit is kept for negative values and -0.0 (a negative value that rounds to zero gives 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    neg = np.signbit(x)
    codes = np.zeros(x.shape, dtype=np.int64)
    # subnormal range: multiples of 2^-9 (q = 8 is the smallest normal, code 0x08, and fits too)
    small = a < 2.0 ** -6
    codes = np.where(small, np.rint(a * 2.0 ** 9), codes)
    # normal range: a = mant * 2^ex with mant in [0.5, 1); unbiased exponent E = ex - 1
    big = (~small) & (a < 464.0)
    _, ex = np.frexp(np.where(big, a, 1.0))
    E = ex - 1
    q = np.rint(np.where(big, a, 1.0) * np.exp2(3.0 - E))  # exact scaling by a power of two
    roll = q >= 16.0
    E = np.where(roll, E + 1, E)
    q = np.where(roll, 8.0, q)
    codes = np.where(big, ((E + 7) << 3) + (q.astype(np.int64) - 8), codes)
    codes = np.where(a >= 464.0, 0x7E, codes).astype(np.int64)  # saturate (448)
    codes = codes | np.where(neg, 0x80, 0).astype(np.int64)
    codes = np.where(np.isnan(x), _E4M3_NAN, codes)
    return codes.astype(np.uint8)


def fwht_f32(y) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform y -> y H_d along the last axis, in float32.

    Butterfly stages with stride h = 1, 2, ..., d/2; each stage replaces the pair (a, b) at positions
    (i, i + h) of every 2h-block by (a + b, a - b).  d must be a power of two.
    """
    y = np.asarray(y, dtype=np.float32)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("Walsh-Hadamard transform needs a power-of-two length")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        t = y.reshape(lead + (d // (2 * h), 2, h))
        a = t[..., 0, :]
        b = t[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return y


def fp8_prep_ref(x, signs, block: int):
    """Block absmax e4m3 quantisation of x [BH, N, d] (or [B, H, N, d]), optionally rotated.

    signs: None (no rotation) or a length-d +/-1 vector.  Returns (codes uint8 same shape as x,
    scales float32 [..., ceil(N / block)]).
    """
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    x = np.asarray(x, dtype=np.float32)
    n, d = x.shape[-2], x.shape[-1]
    lead = x.shape[:-2]
    if signs is not None:
        s = np.asarray(signs).astype(np.float32)
        z = fwht_f32(x * s)
        rs = np.float32(1.0 / np.sqrt(np.float64(d)))
        z = (z * rs).astype(np.float32)
    else:
        z = x
    nblk = -(-n // block)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(lead + (nblk,), dtype=np.float32)
    for bi in range(nblk):
        r0, r1 = bi * block, min(n, (bi + 1) * block)
        zb = z[..., r0:r1, :]
        amax = np.abs(zb).max(axis=(-2, -1)).astype(np.float32)  # [lead]
        zero = amax == 0
        safe = np.where(zero, np.float32(1.0), amax)
        with np.errstate(over="ignore"):
            inv = np.minimum(np.float32(E4M3_MAX) / safe, _F32_MAX).astype(np.float32)
        sc = (safe / np.float32(E4M3_MAX)).astype(np.float32)
        scaled = (zb * inv[..., None, None]).astype(np.float32)
        cb = e4m3_encode(scaled)
        cb = np.where(zero[..., None, None], np.uint8(0), cb)
        codes[..., r0:r1, :] = cb
        scales[..., bi] = np.where(zero, np.float32(1.0), sc)
    return codes, scales


def dequantize_blocks(codes, scales, block: int) -> np.ndarray:
    """code * scale[row // block] in float64, shape of ``codes``."""
    vals = e4m3_decode(codes)
    n = vals.shape[-2]
    sc = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)[..., :n]
    return vals * sc[..., None]


def fp8_attention_ref(q8, sq, k8, sk, v8, sv, block: int, causal: bool, scale: float):
    """Attention in float64 on the dequantised fp8 inputs (what the fp8 kernel approximates)."""
    qd = dequantize_blocks(q8, sq, block)
    kd = dequantize_blocks(k8, sk, block)
    vd = dequantize_blocks(v8, sv, block)
    return attention_ref(qd, kd, vd, causal, scale)

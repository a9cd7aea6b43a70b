"""Seeded input generator for the attention workloads.

Recipe (the same for every caller):
  * every tensor is drawn from its own counter-free NumPy stream
    ``Generator(PCG64(SeedSequence([seed, stream])))``; stream 0/1/2 = Q/K/V,
    stream 3 + t = outlier positions of tensor t (t = 0, 1, 2 for Q, K, V), stream 4 = the +/-1
    sign vector of the head-dimension rotation (only 3 + t for t = 0..2 and 4 are used, so the
    outlier stream of V (5) never collides with the sign stream (4));
  * values are i.i.d. standard normal drawn in float32;
  * for the outlier workload a fixed fraction of flat positions per tensor, chosen uniformly without
    replacement, is multiplied by a constant before rounding;
  * the float32 values are rounded to the storage dtype with round-to-nearest-even (torch's own
    conversion).  The rounded tensors are "the generated inputs": the GPU receives exactly these
    bits and the oracle upcasts exactly these values.

The five named workloads are the attention shapes the method is measured on (tiny fp32 case,
bf16 non-causal, bf16 causal long context, fp16 causal with head dim 256, fp8 with outliers).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

_TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
}


@dataclass(frozen=True)
class Workload:
    """One attention workload: shape, storage dtype, masking and value recipe."""

    cfg_id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32", "f16", "bf16", or "fp8" (fp8: bf16 source tensors quantised on the GPU)
    causal: bool
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    fp8_block: int = 64
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d) rounded to float32 (the value both sides receive)."""
        return float(np.float32(1.0 / np.sqrt(np.float64(self.d))))

    @property
    def flops(self) -> float:
        """Metric flops 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f


WORKLOADS = {
    1: Workload(1, "tiny fp32 SDPA fwd B1 H1 N128 d64 non-causal", 1, 1, 128, 64, "f32", False),
    2: Workload(2, "bf16 SDPA fwd B16 H16 N1024 d128 non-causal", 16, 16, 1024, 128, "bf16", False),
    3: Workload(3, "bf16 causal SDPA fwd B2 H16 N8192 d128", 2, 16, 8192, 128, "bf16", True),
    4: Workload(4, "fp16 causal SDPA fwd B1 H8 N16384 d256", 1, 8, 16384, 256, "f16", True),
    5: Workload(5, "fp8 e4m3 SDPA fwd B4 H16 N4096 d128 non-causal, 0.1% x20 outliers",
                4, 16, 4096, 128, "fp8", False, outlier_frac=0.001, outlier_mult=20.0),
}


def workload(cfg_id: int) -> Workload:
    return WORKLOADS[cfg_id]


def _rng(seed: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream), *sub])))


def normal_f32(shape, seed: int, stream: int) -> np.ndarray:
    """i.i.d. N(0,1) float32 array from the (seed, stream) generator."""
    return _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)


def _apply_outliers(x: np.ndarray, frac: float, mult: float, seed: int, tensor_idx: int) -> np.ndarray:
    if frac <= 0.0:
        return x
    flat = x.reshape(-1)
    count = int(round(frac * flat.size))
    if count == 0:
        return x
    idx = _rng(seed, 3 + tensor_idx).choice(flat.size, size=count, replace=False)
    flat[idx] *= np.float32(mult)
    return x


def gen_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
            outlier_frac: float = 0.0, outlier_mult: float = 1.0):
    """Return (q, k, v) as contiguous CPU torch tensors [B, H, N, d] in the storage dtype.

    ``dtype`` is "f32", "f16" or "bf16"; for the fp8 path pass "bf16" (the source precision).
    """
    tdt = _TORCH_DTYPES[dtype]
    out = []
    for t in range(3):
        x = normal_f32((B, H, N, d), seed, t)
        x = _apply_outliers(x, outlier_frac, outlier_mult, seed, t)
        out.append(torch.from_numpy(x).to(tdt).contiguous())
    return tuple(out)


def gen_qkv_device(B: int, H: int, N: int, d: int, dtype: str, seed: int, device, count: int = 3):
    """``count`` tensors [B, H, N, d] drawn directly in device memory, for shapes too large to draw
    on the host in reasonable time (billions of elements).

    Recipe: tensor t comes from torch's generator of that device seeded with ``seed * 16 + t``,
    i.i.d. standard normal in float32, rounded to the storage dtype.  Repeatable for a given device
    type and torch build; the oracle's side copies the generated (rounded) values it needs back to
    the host, so both sides still see the same bits.
    """
    tdt = _TORCH_DTYPES[dtype]
    out = []
    for t in range(count):
        g = torch.Generator(device=device).manual_seed(int(seed) * 16 + t)
        x = torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32)
        out.append(x.to(tdt))
        del x
    return tuple(out)


def gen_signs(d: int, seed: int) -> np.ndarray:
    """Random +/-1 vector (int8, length d) for the head-dimension rotation."""
    bits = _rng(seed, 4).integers(0, 2, size=d, dtype=np.int8)
    return (bits * 2 - 1).astype(np.int8)


def gen_fp8_workload(w: Workload, seed: int | None = None):
    """bf16 sources (with outliers) plus the sign vector for the fp8 workload."""
    s = w.cfg_id if seed is None else seed
    q, k, v = gen_qkv(w.B, w.H, w.N, w.d, "bf16", s, w.outlier_frac, w.outlier_mult)
    return q, k, v, gen_signs(w.d, s)

"""GPU parity of the attention backward (fa_bwd, through the C ABI) against the float64 oracle.

Tolerance (derived, not printed on the pages): the kernels round P and dS to the 16-bit operand type
(unit roundoff u = 2^-8 for bfloat16, 2^-11 for float16), read o in that type, and accumulate in
float32; each gradient is a sum of such rounded products, so its error relative to the gradient's
own scale stays at a few u.  The bar is max|d - d_ref| <= 5 u * max|d_ref| per dtype: 1.95e-2 for
bfloat16 and 2.44e-3 for float16.
"""

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_bwd_rows
from synth import gen_qkv

pytestmark = pytest.mark.gpu

REL = {"bf16": 5 * 2.0 ** -8, "f16": 5 * 2.0 ** -11}


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


def _inputs(B, H, N, d, dtype, seed):
    q, k, v = gen_qkv(B, H, N, d, dtype, seed=seed)
    do, _, _ = gen_qkv(B, H, N, d, dtype, seed=seed + 1000)
    return q, k, v, do


def _gpu_bwd(q, k, v, do, causal, scale):
    fa = _fa()
    dev = torch.device("cuda")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)]


def _check(got, ref, label, dtype):
    bar = REL[dtype]
    worst = 0.0
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(g).all(), f"{label} {name} not finite"
        err = float(np.abs(g - r).max())
        scale = float(np.abs(r).max())
        rel = err / max(scale, 1e-30)
        worst = max(worst, rel)
        print(f"{label} {name}: max|err| {err:.3e}  max|ref| {scale:.3e}  ratio {rel:.3e}", flush=True)
        assert err <= bar * scale + 1e-6, f"{label} {name}: {err} > {bar} * {scale}"
    return worst


CASES = [
    ("bf16", 128, 1, False), ("bf16", 128, 17, True), ("bf16", 128, 64, False), ("bf16", 128, 100, True),
    ("bf16", 128, 257, False), ("bf16", 128, 300, True), ("bf16", 64, 130, True), ("bf16", 64, 200, False),
    ("f16", 128, 200, False), ("f16", 128, 333, True), ("f16", 64, 96, True),
    ("bf16", 256, 100, True), ("f16", 256, 130, False), ("bf16", 256, 65, False), ("f16", 256, 257, True),
]


@pytest.mark.parametrize("dtype,d,N,causal", CASES)
def test_bwd_sweep(dtype, d, N, causal):
    q, k, v, do = _inputs(2, 2, N, d, dtype, seed=N + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = _gpu_bwd(q, k, v, do, causal, scale)
    ref = attention_bwd_ref(q, k, v, do, causal, scale)
    _check(got, ref, f"{dtype} d{d} N{N} causal={causal}", dtype)


def test_bwd_negative_scale_and_determinism():
    q, k, v, do = _inputs(1, 2, 150, 128, "bf16", seed=9)
    scale = -float(np.float32(1 / np.sqrt(128)))
    a = _gpu_bwd(q, k, v, do, False, scale)
    b = _gpu_bwd(q, k, v, do, False, scale)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "backward is not bitwise repeatable"
    _check(a, attention_bwd_ref(q, k, v, do, False, scale), "negative scale", "bf16")


@pytest.mark.parametrize("d,causal", [(64, True), (128, True), (256, False), (256, True)])
@pytest.mark.parametrize("kind", ["negative", "zero"])
def test_bwd_negative_and_zero_scale_masks(d, causal, kind):
    # hidden keys (causal, and the rows past N of a ragged last tile) must get weight 0 whatever the
    # scale's sign; with scale 0 every visible key of a row gets the same weight
    q, k, v, do = _inputs(1, 2, 150, d, "bf16", seed=11 + d)
    scale = -float(np.float32(1 / np.sqrt(d))) if kind == "negative" else 0.0
    got = _gpu_bwd(q, k, v, do, causal, scale)
    _check(got, attention_bwd_ref(q, k, v, do, causal, scale), f"{kind} scale d{d} causal={causal}", "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_full_size_sampled_heads(causal):
    # B16 H16 N1024 d128 in one launch; four heads checked against the oracle
    B, H, N, d = 16, 16, 1024, 128
    q, k, v, do = _inputs(B, H, N, d, "bf16", seed=21)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = _gpu_bwd(q, k, v, do, causal, scale)
    rng = np.random.default_rng(4)
    for bh in rng.choice(B * H, size=4, replace=False):
        b, h = divmod(int(bh), H)
        ref = attention_bwd_rows(q[b, h], k[b, h], v[b, h], do[b, h], causal, scale)
        _check([g[b, h] for g in got], ref, f"B16H16N1024 head {b},{h} causal={causal}", "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_d256_long_sampled_heads(causal):
    # d = 256 at a longer sequence (fp16, the large-head forward workload's dtype; both masks)
    B, H, N, d = 1, 2, 4096, 256
    q, k, v, do = _inputs(B, H, N, d, "f16", seed=31)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = _gpu_bwd(q, k, v, do, causal, scale)
    for h in range(H):
        ref = attention_bwd_rows(q[0, h], k[0, h], v[0, h], do[0, h], causal, scale)
        _check([g[0, h] for g in got], ref, f"f16 d256 N{N} head {h} causal={causal}", "f16")

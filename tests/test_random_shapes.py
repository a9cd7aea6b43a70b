"""GPU parity of the forward and backward kernels on seeded random shapes (ragged query and key tiles, every head
dimension, both masks, B*H above one), against the float64 CPU oracle through the C ABI.

Tolerances as for the fixed sweeps: max|dO| <= 1e-2 and max|dlse| <= 1e-3 for float16/bfloat16 with
N(0,1) inputs; RMSE(O) <= 3e-2 against the dequantised-input oracle for the e4m3 path (plus max|dlse|
<= 1e-3 there too, as the fixed fp8 cases check).
"""

import math

import numpy as np
import pytest
import torch

from bars import LSE_BAR, o_bar
from oracle import attention_ref, fp8_attention_ref, fp8_prep_ref
from synth import gen_qkv, gen_signs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


def _cases16(n=18, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        # keep the oracle cheap: B*H*N^2*d below ~3e9 multiply-adds
        N = int(rng.integers(1, 2400 if d < 256 else 1400))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        out.append((str(rng.choice(["bf16", "f16"])), d, B, H, N, bool(rng.integers(0, 2)), 5000 + i))
    return out


def _cases8(n=8, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        N = int(rng.integers(1, 1500))
        out.append((d, int(rng.integers(1, 3)), N, bool(rng.integers(0, 2)), 6000 + i))
    return out


@pytest.mark.parametrize("dtype,d,B,H,N,causal,seed", _cases16())
def test_random_shape_16bit(dtype, d, B, H, N, causal, seed):
    import exact_tiled_attention_22_amd as fa

    q, k, v = gen_qkv(B, H, N, d, dtype, seed=seed)
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = torch.device("cuda")
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    o_ref, lse_ref = attention_ref(q, k, v, causal, scale)
    do = float(np.abs(o - o_ref).max())
    dl = float(np.abs(lse - lse_ref).max())
    print(f"{dtype} d{d} B{B} H{H} N{N} causal={causal}: max|dO|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert do <= TOL_O and dl <= TOL_LSE
    assert do <= o_bar(dtype, v) and dl <= LSE_BAR  # the dtype's own bar (bars.py)


@pytest.mark.parametrize("d,H,N,causal,seed", _cases8())
def test_random_shape_fp8(d, H, N, causal, seed):
    import exact_tiled_attention_22_amd as fa

    q, k, v = gen_qkv(1, H, N, d, "bf16", seed=seed, outlier_frac=0.001, outlier_mult=20.0)
    signs = gen_signs(d, seed=seed)
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = torch.device("cuda")
    q8, sq = fa.fp8_prep(q.to(dev), signs, 64)
    k8, sk = fa.fp8_prep(k.to(dev), signs, 64)
    v8, sv = fa.fp8_prep(v.to(dev), None, 64)
    o, lse = fa.fwd(q8, k8, v8, causal=causal, scale=scale, fp8_scales=(sq, sk, sv))
    torch.cuda.synchronize()
    cq, csq = fp8_prep_ref(q, signs, 64)
    ck, csk = fp8_prep_ref(k, signs, 64)
    cv, csv = fp8_prep_ref(v, None, 64)
    o_ref, lse_ref = fp8_attention_ref(cq, csq, ck, csk, cv, csv, 64, causal, scale)
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rmse = float(np.sqrt(np.mean((o.astype(np.float64) - o_ref) ** 2)))
    dl = float(np.abs(lse - lse_ref).max())
    print(f"fp8 d{d} H{H} N{N} causal={causal}: RMSE {rmse:.3e} max|dlse|={dl:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert rmse <= 3e-2 and dl <= TOL_LSE


def _cases_bwd(n=12, seed=2028):
    # the backward kernels unroll six tiles with a guarded tail: N covers many residues of the tile count
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        N = int(rng.integers(1, 1100 if d < 256 else 700))
        out.append((str(rng.choice(["bf16", "f16"])), d, int(rng.integers(1, 3)), int(rng.integers(1, 3)), N,
                    bool(rng.integers(0, 2)), 7000 + i))
    return out


@pytest.mark.parametrize("dtype,d,B,H,N,causal,seed", _cases_bwd())
def test_random_shape_backward(dtype, d, B, H, N, causal, seed):
    import exact_tiled_attention_22_amd as fa
    from oracle import attention_bwd_ref

    q, k, v = gen_qkv(B, H, N, d, dtype, seed=seed)
    do = gen_qkv(B, H, N, d, dtype, seed=seed + 100)[0]
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = torch.device("cuda")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    got = [t.float().cpu().numpy() for t in fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)]
    ref = attention_bwd_ref(q, k, v, do, causal, scale)
    # per-gradient bar from the operand type's rounding, as in the fixed backward sweep
    bar = 5 * 2.0 ** (-8 if dtype == "bf16" else -11)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        err, top = float(np.abs(g - r).max()), float(np.abs(r).max())
        print(f"bwd {dtype} d{d} B{B} H{H} N{N} causal={causal} {name}: max|err| {err:.3e} max|ref| {top:.3e}",
              flush=True)
        assert np.isfinite(g).all() and err <= bar * top + 1e-6

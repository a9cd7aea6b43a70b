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
from oracle import attention_rect, attention_ref, fp8_attention_ref, fp8_prep_ref
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


def _cases_rect(n=16, seed=2029):
    # queries at a random position of a longer key sequence: rectangular, key-split and decode calls
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        Nk = int(rng.integers(1, 2500 if d < 256 else 1500))
        Nq = int(rng.integers(1, Nk + 1))
        causal = bool(rng.integers(0, 2))
        q_start = int(rng.integers(0, Nk - Nq + 1)) if causal else 0
        out.append((str(rng.choice(["bf16", "f16"])), d, int(rng.integers(1, 3)), int(rng.integers(1, 3)), Nq, Nk,
                    q_start, causal, int(rng.integers(1, 9)), 7000 + i))
    return out


def _check_rect(o, lse, q, k, v, causal, scale, q_start, dtype, label):
    B, H = q.shape[:2]
    wo = wl = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, lse_ref = attention_rect(q[b, h], k[b, h], v[b, h], causal, scale, q_start=q_start)
            wo = max(wo, float(np.abs(o[b, h] - o_ref).max()))
            wl = max(wl, float(np.abs(lse[b, h] - lse_ref).max()))
    print(f"{label}: max|dO|={wo:.3e} max|dlse|={wl:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), label
    assert wo <= TOL_O and wo <= o_bar(dtype, v), label
    assert wl <= TOL_LSE and wl <= LSE_BAR, label


@pytest.mark.parametrize("dtype,d,B,H,Nq,Nk,q_start,causal,nsplit,seed", _cases_rect())
def test_random_shape_rect_and_split(dtype, d, B, H, Nq, Nk, q_start, causal, nsplit, seed):
    import exact_tiled_attention_22_amd as fa

    q = gen_qkv(B, H, Nq, d, dtype, seed=seed)[0]
    _, k, v = gen_qkv(B, H, Nk, d, dtype, seed=seed + 1)
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    label = f"{dtype} d{d} B{B} H{H} Nq{Nq} Nk{Nk} q_start{q_start} causal={causal}"
    o, lse = fa.fwd_rect(qd, kd, vd, causal=causal, q_start=q_start, scale=scale)
    _check_rect(o.float().cpu().numpy(), lse.cpu().numpy(), q, k, v, causal, scale, q_start, dtype, "rect " + label)
    o, lse = fa.fwd_split(qd, kd, vd, nsplit=nsplit, causal=causal, q_start=q_start, scale=scale)
    _check_rect(o.float().cpu().numpy(), lse.cpu().numpy(), q, k, v, causal, scale, q_start, dtype,
                f"split{nsplit} " + label)


def _cases_decode(n=16, seed=2030):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        Nq = int(rng.choice([1, 1, int(rng.integers(2, 33))]))
        Nk = int(rng.integers(Nq, 20000 if d < 256 else 8000))
        out.append((str(rng.choice(["bf16", "f16"])), d, int(rng.integers(1, 3)), int(rng.integers(1, 5)), Nq, Nk,
                    bool(rng.integers(0, 2)), 8000 + i))
    return out


@pytest.mark.parametrize("dtype,d,B,H,Nq,Nk,causal,seed", _cases_decode())
def test_random_shape_decode(dtype, d, B, H, Nq, Nk, causal, seed):
    import exact_tiled_attention_22_amd as fa

    qf, k, v = gen_qkv(B, H, Nk, d, dtype, seed=seed)
    q = qf[:, :, Nk - Nq:].contiguous()  # the last Nq positions
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = torch.device("cuda")
    o, lse = fa.fwd_decode(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    _check_rect(o.float().cpu().numpy(), lse.cpu().numpy(), q, k, v, causal, scale, Nk - Nq, dtype,
                f"decode {dtype} d{d} B{B} H{H} Nq{Nq} Nk{Nk} causal={causal}")

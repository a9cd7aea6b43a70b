"""Ragged-tail sweeps on the GPU, each case against the float64 oracle.

The tile loops meet a partial last tile of keys (64 keys for 16-bit d <= 128, 32 for d = 256 and float32) and a partial last
tile of query rows; the backward kernels unroll six tiles and finish with a guarded tail.  These sweeps
walk every sequence length up to a little past one tile (so every residue of the key-tile size) for the
forward, and sequence lengths whose tile counts cover every position of the six-tile unroll for the
backward, with the bars of the fixed sweeps (tests/bars.py; the backward's per-dtype relative bar).
"""
import math

import numpy as np
import pytest
import torch

from bars import LSE_BAR, STATED_LSE, STATED_O, o_bar
from oracle import attention_bwd_ref, attention_ref, fp8_attention_ref, fp8_prep_ref
from synth import gen_qkv, gen_signs

pytestmark = pytest.mark.gpu

BWD_REL = {"bf16": 5 * 2.0 ** -8, "f16": 5 * 2.0 ** -11}


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


def _scale(d):
    return float(np.float32(1 / math.sqrt(d)))


@pytest.mark.parametrize("dtype,d,causal,Ns", [
    ("bf16", 128, False, range(1, 130)), ("bf16", 128, True, range(1, 130)),
    ("f16", 256, False, range(1, 98)), ("f16", 256, True, range(1, 98)),
    ("f16", 64, True, range(1, 130, 2)),
])
def test_forward_every_tail_length(dtype, d, causal, Ns):
    fa = _fa()
    dev = torch.device("cuda")
    worst_o = worst_l = 0.0
    for N in Ns:
        q, k, v = gen_qkv(1, 2, N, d, dtype, seed=31 * N + d)
        o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=_scale(d))
        torch.cuda.synchronize()
        o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
        o_ref, lse_ref = attention_ref(q, k, v, causal, _scale(d))
        do, dl = float(np.abs(o - o_ref).max()), float(np.abs(lse - lse_ref).max())
        label = f"{dtype} d{d} causal={causal} N{N}: max|dO|={do:.3e} max|dlse|={dl:.3e}"
        assert np.isfinite(o).all() and np.isfinite(lse).all(), label
        assert do <= STATED_O and do <= o_bar(dtype, v) and dl <= STATED_LSE and dl <= LSE_BAR, label
        worst_o, worst_l = max(worst_o, do), max(worst_l, dl)
    print(f"{dtype} d{d} causal={causal} N {Ns.start}..{Ns.stop - 1}: worst max|dO|={worst_o:.3e} "
          f"max|dlse|={worst_l:.3e}", flush=True)


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True), (256, True)])
def test_fp32_forward_tail_lengths(d, causal):
    # float32 kernel: 32-key tiles and 128-row query tiles; N = 1..70 meets every residue of the key tile
    # (twice), and the lengths around 128 and 256 the partial and full second and third query tiles
    fa = _fa()
    dev = torch.device("cuda")
    worst_o = worst_l = 0.0
    for N in list(range(1, 71)) + [126, 127, 128, 129, 130, 255, 256, 257]:
        q, k, v = gen_qkv(1, 2, N, d, "f32", seed=13 * N + d)
        o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=_scale(d))
        torch.cuda.synchronize()
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        o_ref, lse_ref = attention_ref(q, k, v, causal, _scale(d))
        do, dl = float(np.abs(o - o_ref).max()), float(np.abs(lse - lse_ref).max())
        label = f"f32 d{d} causal={causal} N{N}: max|dO|={do:.3e} max|dlse|={dl:.3e}"
        assert np.isfinite(o).all() and np.isfinite(lse).all(), label
        assert do <= o_bar("f32", v) and dl <= LSE_BAR, label
        worst_o, worst_l = max(worst_o, do), max(worst_l, dl)
    print(f"f32 d{d} causal={causal}: worst max|dO|={worst_o:.3e} max|dlse|={worst_l:.3e}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_every_tail_length(causal):
    fa = _fa()
    dev = torch.device("cuda")
    d = 128
    signs = gen_signs(d, seed=d)
    worst = 0.0
    for N in range(1, 130):
        q, k, v = gen_qkv(1, 2, N, d, "bf16", seed=17 * N, outlier_frac=0.001, outlier_mult=20.0)
        q8, sq = fa.fp8_prep(q.to(dev), signs, 64)
        k8, sk = fa.fp8_prep(k.to(dev), signs, 64)
        v8, sv = fa.fp8_prep(v.to(dev), None, 64)
        o, lse = fa.fwd(q8, k8, v8, causal=causal, scale=_scale(d), fp8_scales=(sq, sk, sv))
        torch.cuda.synchronize()
        cq, csq = fp8_prep_ref(q, signs, 64)
        ck, csk = fp8_prep_ref(k, signs, 64)
        cv, csv = fp8_prep_ref(v, None, 64)
        o_ref, lse_ref = fp8_attention_ref(cq, csq, ck, csk, cv, csv, 64, causal, _scale(d))
        o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
        rmse = float(np.sqrt(np.mean((o.astype(np.float64) - o_ref) ** 2)))
        dl = float(np.abs(lse - lse_ref).max())
        label = f"e4m3 d{d} causal={causal} N{N}: RMSE {rmse:.3e} max|dlse|={dl:.3e}"
        assert np.isfinite(o).all() and rmse <= 3e-2 and dl <= 1e-3, label
        worst = max(worst, rmse)
    print(f"e4m3 d{d} causal={causal} N 1..129: worst RMSE {worst:.3e}", flush=True)


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (256, False), (256, True)])
def test_fp8_forward_tail_lengths_other_dims(d, causal):
    # 64-key tiles; 128-row (d = 64) and 256-row (d = 256) query tiles
    fa = _fa()
    dev = torch.device("cuda")
    signs = gen_signs(d, seed=d)
    worst = 0.0
    for N in list(range(1, 71)) + [127, 128, 129, 255, 256, 257]:
        q, k, v = gen_qkv(1, 2, N, d, "bf16", seed=19 * N + d, outlier_frac=0.001, outlier_mult=20.0)
        q8, sq = fa.fp8_prep(q.to(dev), signs, 64)
        k8, sk = fa.fp8_prep(k.to(dev), signs, 64)
        v8, sv = fa.fp8_prep(v.to(dev), None, 64)
        o, lse = fa.fwd(q8, k8, v8, causal=causal, scale=_scale(d), fp8_scales=(sq, sk, sv))
        torch.cuda.synchronize()
        cq, csq = fp8_prep_ref(q, signs, 64)
        ck, csk = fp8_prep_ref(k, signs, 64)
        cv, csv = fp8_prep_ref(v, None, 64)
        o_ref, lse_ref = fp8_attention_ref(cq, csq, ck, csk, cv, csv, 64, causal, _scale(d))
        o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
        rmse = float(np.sqrt(np.mean((o.astype(np.float64) - o_ref) ** 2)))
        dl = float(np.abs(lse - lse_ref).max())
        label = f"e4m3 d{d} causal={causal} N{N}: RMSE {rmse:.3e} max|dlse|={dl:.3e}"
        assert np.isfinite(o).all() and rmse <= 3e-2 and dl <= 1e-3, label
        worst = max(worst, rmse)
    print(f"e4m3 d{d} causal={causal}: worst RMSE {worst:.3e}", flush=True)


def _bwd_lengths(t_max):
    # 32-row query tiles (dK/dV loop) and 64-key tiles (dQ loop): t full tiles plus 1 or 31 rows
    return sorted({32 * t + r for t in range(t_max) for r in (1, 31)})


@pytest.mark.parametrize("dtype,d,causal,t_max", [
    ("bf16", 128, True, 28), ("bf16", 128, False, 28), ("f16", 64, True, 28), ("f16", 256, True, 14),
])
def test_backward_every_unroll_position(dtype, d, causal, t_max):
    fa = _fa()
    dev = torch.device("cuda")
    bar = BWD_REL[dtype]
    worst = 0.0
    for N in _bwd_lengths(t_max):
        q, k, v = gen_qkv(1, 1, N, d, dtype, seed=7 * N + d)
        do, _, _ = gen_qkv(1, 1, N, d, dtype, seed=7 * N + d + 1000)
        qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
        o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=_scale(d))
        got = [t.float().cpu().numpy() for t in fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=_scale(d))]
        torch.cuda.synchronize()
        ref = attention_bwd_ref(q, k, v, do, causal, _scale(d))
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            err, top = float(np.abs(g - r).max()), float(np.abs(r).max())
            label = f"{dtype} d{d} causal={causal} N{N} {name}: max|err| {err:.3e} max|ref| {top:.3e}"
            assert np.isfinite(g).all() and err <= bar * top + 1e-6, label
            worst = max(worst, err / max(top, 1e-3))  # (N = 1 causal: dq = dk = 0 exactly)
    print(f"bwd {dtype} d{d} causal={causal} N 1..{32 * t_max - 1}: worst max|err|/max|ref| {worst:.3e}",
          flush=True)

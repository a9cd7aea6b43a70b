"""GPU parity of the fp8 preparation kernel (bitwise) and the fp8 forward (RMSE) against the oracle."""

import numpy as np
import pytest
import torch

from oracle import (
    attention_ref,
    attention_rows,
    dequantize_blocks,
    e4m3_decode,
    e4m3_encode,
    fp8_attention_ref,
    fp8_prep_ref,
)
from synth import WORKLOADS, gen_fp8_workload, gen_qkv, gen_signs

pytestmark = pytest.mark.gpu


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("rotate", [False, True])
def test_prep_bitwise(dtype, d, rotate):
    fa = _fa()
    N, block = 200, 64  # three full blocks and a partial one
    q, _, _ = gen_qkv(1, 3, N, d, dtype, seed=d + 1, outlier_frac=0.002, outlier_mult=20.0)
    signs = gen_signs(d, seed=d) if rotate else None
    codes, scales = fa.fp8_prep(q.cuda(), signs, block)
    torch.cuda.synchronize()
    c_ref, s_ref = fp8_prep_ref(q, signs, block)
    got = codes.view(torch.uint8).cpu().numpy()
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    mism = got != c_ref
    print(f"prep {dtype} d{d} rotate={rotate}: {int(mism.sum())} code mismatches", flush=True)
    np.testing.assert_array_equal(got, c_ref)


@pytest.mark.parametrize("block", [1, 16, 100, 1024])
def test_prep_other_blocks_and_zero_block(block):
    fa = _fa()
    q, _, _ = gen_qkv(1, 2, 300, 128, "bf16", seed=block)
    q[0, 1, :block] = 0  # first block of the second head is all zero
    codes, scales = fa.fp8_prep(q.cuda(), gen_signs(128, 3), block)
    torch.cuda.synchronize()
    c_ref, s_ref = fp8_prep_ref(q, gen_signs(128, 3), block)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.view(torch.uint8).cpu().numpy(), c_ref)


@pytest.mark.parametrize("dtype,d,N,block,rotate", [("bf16", 128, 4096, 64, True), ("bf16", 64, 200, 64, True),
                                                    ("f16", 256, 333, 64, True), ("f32", 128, 130, 100, False)])
def test_prep_qkv_one_launch_bitwise(dtype, d, N, block, rotate):
    # one launch for Q, K (rotated with the shared signs) and V (not rotated): bitwise the three
    # separate preparations and the oracle's model
    fa = _fa()
    q, k, v = gen_qkv(2, 3, N, d, dtype, seed=d + N, outlier_frac=0.001, outlier_mult=20.0)
    signs = gen_signs(d, seed=d) if rotate else None
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    fused = fa.fp8_prep_qkv(qd, kd, vd, signs, block)
    apart = (fa.fp8_prep(qd, signs, block), fa.fp8_prep(kd, signs, block), fa.fp8_prep(vd, None, block))
    torch.cuda.synchronize()
    for name, x, (c8, sc), (a8, asc), sg in zip("qkv", (q, k, v), fused, apart, (signs, signs, None)):
        assert torch.equal(c8.view(torch.uint8), a8.view(torch.uint8)) and torch.equal(sc, asc), name
        c_ref, s_ref = fp8_prep_ref(x, sg, block)
        np.testing.assert_array_equal(c8.view(torch.uint8).cpu().numpy(), c_ref)
        np.testing.assert_array_equal(sc.cpu().numpy(), s_ref)
    print(f"prep qkv {dtype} d{d} N{N} block{block} rotate={rotate}: bitwise equal", flush=True)


def _rmse(a, b):
    return float(np.sqrt(np.mean((np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)) ** 2)))


def _fp8_case(B, H, N, d, causal, seed, outliers=True, scale=None):
    fa = _fa()
    frac, mult = (0.001, 20.0) if outliers else (0.0, 1.0)
    q, k, v = gen_qkv(B, H, N, d, "bf16", seed=seed, outlier_frac=frac, outlier_mult=mult)
    signs = gen_signs(d, seed=seed)
    scale = float(np.float32(1 / np.sqrt(d))) if scale is None else scale
    dev = torch.device("cuda")
    q8, sq = fa.fp8_prep(q.to(dev), signs, 64)
    k8, sk = fa.fp8_prep(k.to(dev), signs, 64)
    v8, sv = fa.fp8_prep(v.to(dev), None, 64)
    o, lse = fa.fwd(q8, k8, v8, causal=causal, scale=scale, fp8_scales=(sq, sk, sv))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    # oracle (i): its own quantisation of the same bf16 inputs, then float64 attention
    cq, csq = fp8_prep_ref(q, signs, 64)
    ck, csk = fp8_prep_ref(k, signs, 64)
    cv, csv = fp8_prep_ref(v, None, 64)
    o_i, lse_i = fp8_attention_ref(cq, csq, ck, csk, cv, csv, 64, causal, scale)
    o_ii, _ = attention_ref(q, k, v, causal, scale)  # (ii): original inputs
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    r_i, r_ii = _rmse(o, o_i), _rmse(o, o_ii)
    floor = _rmse(o_i, o_ii)
    dl = float(np.abs(lse - lse_i).max())
    print(f"fp8 B{B} H{H} N{N} d{d} causal={causal}: RMSE vs dequantised-input oracle {r_i:.3e}, "
          f"vs original inputs {r_ii:.3e} (format floor {floor:.3e}), max|dlse| {dl:.2e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    return r_i, r_ii, dl


@pytest.mark.parametrize("N,d,causal", [(200, 128, False), (333, 128, True), (64, 64, False), (130, 64, True),
                                        (256, 256, False), (300, 256, True), (1, 128, False)])
def test_fp8_forward_rmse(N, d, causal):
    r_i, _, dl = _fp8_case(1, 2, N, d, causal, seed=N + d)
    assert r_i <= 3e-2
    assert dl <= 1e-3
    # the kernel's own error budget (rows of a single key or of 64+ keys measure 1.6e-3 .. 5.3e-3; rows
    # of only a dozen keys, as in the random-shape tests, reach about 8e-3 and keep the format's bar)
    assert r_i <= 8e-3


def test_fp8_forward_unit_scales_and_negative_scale():
    fa = _fa()
    # codes used directly (no scales): value = code; N(0,1) values rounded to e4m3 keep the contract
    rng = np.random.default_rng(3)
    codes = [e4m3_encode(rng.standard_normal((1, 1, 150, 128))) for _ in range(3)]
    t = [torch.from_numpy(c).view(torch.float8_e4m3fn).cuda() for c in codes]
    s0 = float(np.float32(1 / np.sqrt(128)))
    for scale in (s0, -s0):
        o, lse = fa.fwd(*t, causal=False, scale=scale)
        torch.cuda.synchronize()
        vals = [e4m3_decode(c) for c in codes]
        o_ref, lse_ref = attention_ref(*vals, False, scale)
        r = _rmse(o.float().cpu().numpy(), o_ref)
        print(f"fp8 unit scales scale={scale}: RMSE {r:.3e}", flush=True)
        assert r <= 3e-2 and float(np.abs(lse.cpu().numpy() - lse_ref).max()) <= 1e-3


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 4, 300, 128, False), (2, 4, 300, 128, True), (4, 4, 200, 64, True),
                                             (2, 8, 260, 256, False), (1, 8, 130, 256, True), (4, 4, 257, 128, False)])
def test_fp8_xcd_partition_element_wise(B, H, N, d, causal):
    # B*H a multiple of 8 (the work partition's XCD branch), every element against oracle (i)
    r_i, _, dl = _fp8_case(B, H, N, d, causal, seed=B * 100 + H * 10 + N + d)
    assert r_i <= 3e-2 and dl <= 1e-3
    assert r_i <= 8e-3  # the kernel's own error budget


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_zero_v_scale_block(d):
    """A V block whose scale is 0 dequantises to zeros: its keys keep their softmax weight but add no value
    (scales of exactly 0 are never written by the preparation, which gives an all-zero block scale 1)."""
    fa = _fa()
    N = 200
    q, k, v = gen_qkv(1, 2, N, d, "bf16", seed=40 + d)
    signs = gen_signs(d, seed=d)
    dev = torch.device("cuda")
    q8, sq = fa.fp8_prep(q.to(dev), signs, 64)
    k8, sk = fa.fp8_prep(k.to(dev), signs, 64)
    v8, sv = fa.fp8_prep(v.to(dev), None, 64)
    sv[0, 1, 1] = 0.0  # second 64-key block of head 1
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = fa.fwd(q8, k8, v8, causal=False, scale=scale, fp8_scales=(sq, sk, sv))
    torch.cuda.synchronize()
    cq, csq = fp8_prep_ref(q, signs, 64)
    ck, csk = fp8_prep_ref(k, signs, 64)
    cv, csv = fp8_prep_ref(v, None, 64)
    csv[0, 1, 1] = 0.0
    o_i, lse_i = fp8_attention_ref(cq, csq, ck, csk, cv, csv, 64, False, scale)
    o = o.float().cpu().numpy()
    r = _rmse(o, o_i)
    dl = float(np.abs(lse.cpu().numpy() - lse_i).max())
    print(f"fp8 zero V scale d{d}: RMSE {r:.3e}, max|dlse| {dl:.2e}", flush=True)
    assert np.isfinite(o).all() and r <= 3e-2 and dl <= 1e-3


def test_fp8_full_config5_sampled_rows():
    fa = _fa()
    w = WORKLOADS[5]
    q, k, v, signs = gen_fp8_workload(w)
    dev = torch.device("cuda")
    q8, sq = fa.fp8_prep(q.to(dev), signs, 64)
    k8, sk = fa.fp8_prep(k.to(dev), signs, 64)
    v8, sv = fa.fp8_prep(v.to(dev), None, 64)
    o, lse = fa.fwd(q8, k8, v8, causal=w.causal, scale=w.scale, fp8_scales=(sq, sk, sv))
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rng = np.random.default_rng(55)
    err_i, err_ii, worst_l = [], [], 0.0
    dense = set(int(x) for x in rng.choice(w.B * w.H, size=3, replace=False))
    for bh in range(w.B * w.H):
        # every head: 62 random rows on three of them, 6 on the others (the first and last row included)
        b, h = divmod(bh, w.H)
        cq, csq = fp8_prep_ref(q[b, h][None], signs, 64)
        ck, csk = fp8_prep_ref(k[b, h][None], signs, 64)
        cv, csv = fp8_prep_ref(v[b, h][None], None, 64)
        qd, kd, vd = (dequantize_blocks(c, s_, 64)[0] for c, s_ in ((cq, csq), (ck, csk), (cv, csv)))
        rows = np.unique(np.concatenate([[0, w.N - 1], rng.integers(0, w.N, 62 if bh in dense else 4)]))
        o_i, lse_i = attention_rows(qd, kd, vd, rows, w.causal, w.scale)
        o_ii, _ = attention_rows(q[b, h], k[b, h], v[b, h], rows, w.causal, w.scale)
        err_i.append(o[b, h][rows] - o_i)
        err_ii.append(o[b, h][rows] - o_ii)
        worst_l = max(worst_l, float(np.abs(lse[b, h][rows] - lse_i).max()))
    r_i = float(np.sqrt(np.mean(np.concatenate(err_i) ** 2)))
    r_ii = float(np.sqrt(np.mean(np.concatenate(err_ii) ** 2)))
    print(f"{w.name}: sampled RMSE vs dequantised-input oracle {r_i:.3e}, vs original inputs {r_ii:.3e}, "
          f"max|dlse| {worst_l:.2e}", flush=True)
    assert np.isfinite(o).all()
    assert r_i <= 3e-2 and worst_l <= 1e-3
    # the kernel's own error budget on this workload (a regression check beside the 3e-2 contract): a CPU
    # model of the kernel's rounding (exact power-of-two boost of p, V block scale applied in float32,
    # lazy maximum with slack 2^2, bf16 output) gives 4.0e-3 against the dequantised-input oracle
    assert r_i <= 8e-3, f"e4m3 kernel error {r_i:.3e} above its 8e-3 budget"

"""GPU parity of the unfused comparison path (fa_naive_scores -> fa_naive_softmax -> fa_naive_pv, and
fa_fwd_naive) against the float64 oracle: the intermediates S and P against attention_probs, the output
and lse against attention_ref / attention_rows with the forward bar max|dO| <= 1e-2, max|dlse| <= 1e-3."""

import numpy as np
import pytest
import torch

from bars import LSE_BAR, o_bar
from oracle import attention_probs, attention_ref, attention_rows
from synth import gen_qkv

pytestmark = pytest.mark.gpu


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


def _scale(d):
    return float(np.float32(1 / np.sqrt(d)))


CASES = [
    ("bf16", 128, 1, 2, 1, False), ("bf16", 128, 2, 3, 130, True), ("f16", 64, 1, 2, 300, False),
    ("bf16", 256, 1, 1, 200, True), ("f16", 256, 1, 2, 64, False), ("bf16", 64, 2, 2, 1000, True),
    ("f16", 128, 1, 1, 517, True),
]


@pytest.mark.parametrize("dtype,d,B,H,N,causal", CASES)
def test_naive_stages_and_output(dtype, d, B, H, N, causal):
    fa = _fa()
    dev = torch.device("cuda")
    q, k, v = gen_qkv(B, H, N, d, dtype, seed=N + d)
    scale = _scale(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    s = fa.naive_scores(qd, kd, scale=scale)
    p, lse = fa.naive_softmax(s, dtype=qd.dtype, causal=causal)
    o = fa.naive_pv(p, vd)
    o2, lse2 = fa.fwd_naive(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ld = fa.naive_row_stride(N)
    assert s.shape == (B, H, N, ld) and p.shape == (B, H, N, ld)
    s_np, p_np = s.cpu().numpy(), p.float().cpu().numpy()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    # the one-call entry point runs the same three kernels: identical bits
    assert torch.equal(o2.cpu(), o.cpu()) and torch.equal(lse2.cpu(), lse.cpu())
    ws = wp = 0.0
    for b in range(B):
        for h in range(H):
            s_ref, p_ref, _ = attention_probs(q[b, h], k[b, h], causal, scale)
            ds = np.abs(s_np[b, h, :, :N] - s_ref)
            assert (ds <= 1e-5 * (1.0 + np.abs(s_ref))).all(), f"S: max err {ds.max():.3e}"
            dp = np.abs(p_np[b, h, :, :N] - p_ref)
            rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -10
            assert (dp <= rel * p_ref + 1e-6).all(), f"P: max err {dp.max():.3e}"
            assert (p_np[b, h, :, N:] == 0).all()  # padding columns
            if causal:
                assert (p_np[b, h][np.triu_indices(N, 1)] == 0).all()  # masked keys exactly 0
            ws, wp = max(ws, float(ds.max())), max(wp, float(dp.max()))
    o_ref, lse_ref = attention_ref(q, k, v, causal, scale)
    wo, wl = float(np.abs(o_np - o_ref).max()), float(np.abs(lse_np - lse_ref).max())
    print(f"naive {dtype} d{d} B{B} H{H} N{N} causal={causal}: max|dS| {ws:.2e} max|dP| {wp:.2e} "
          f"max|dO| {wo:.3e} max|dlse| {wl:.3e}", flush=True)
    assert np.isfinite(o_np).all() and wo <= 1e-2 and wl <= 1e-3
    assert wo <= o_bar(dtype, v) and wl <= LSE_BAR  # the dtype's own bar (bars.py)


# rows longer than 8192 take the two-pass softmax; full-size workloads are checked on sampled rows
SAMPLED = [
    ("bf16", 64, 1, 1, 9000, False), ("f16", 128, 1, 2, 8300, True),
    ("bf16", 128, 16, 16, 1024, False), ("bf16", 128, 2, 16, 8192, True),
]


@pytest.mark.parametrize("dtype,d,B,H,N,causal", SAMPLED)
def test_naive_sampled_rows(dtype, d, B, H, N, causal):
    fa = _fa()
    dev = torch.device("cuda")
    q, k, v = gen_qkv(B, H, N, d, dtype, seed=7 * N + d)
    scale = _scale(d)
    o, lse = fa.fwd_naive(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(N)
    heads = {(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))}
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 2, N - 1], rng.integers(0, N, 27)]))
    wo = wl = 0.0
    for b, h in sorted(heads):
        o_ref, lse_ref = attention_rows(q[b, h], k[b, h], v[b, h], rows, causal, scale)
        wo = max(wo, float(np.abs(o_np[b, h, rows] - o_ref).max()))
        wl = max(wl, float(np.abs(lse_np[b, h, rows] - lse_ref).max()))
    print(f"naive {dtype} d{d} B{B} H{H} N{N} causal={causal} ({len(rows)} rows x {len(heads)} heads): "
          f"max|dO| {wo:.3e} max|dlse| {wl:.3e}", flush=True)
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    assert wo <= 1e-2 and wl <= 1e-3
    assert wo <= o_bar(dtype, v) and wl <= LSE_BAR  # the dtype's own bar (bars.py)

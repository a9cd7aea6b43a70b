"""GPU parity of the decode path (fa_fwd_decode: few queries against a long key cache, keys split
over waves and merged) against the float64 oracle (attention_rect), with the forward bar:
max|dO| <= 1e-2, max|dlse| <= 1e-3."""

import numpy as np
import pytest
import torch

from bars import LSE_BAR, o_bar
from oracle import attention_rect
from synth import gen_qkv

pytestmark = pytest.mark.gpu


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


def _inputs(B, H, Nq, Nk, d, dtype, seed):
    # the queries are the last Nq positions of a sequence of Nk
    qf, k, v = gen_qkv(B, H, Nk, d, dtype, seed=seed)
    return qf[:, :, Nk - Nq:, :].contiguous(), k, v


def _run(q, k, v, causal, scale):
    fa = _fa()
    dev = torch.device("cuda")
    o, lse = fa.fwd_decode(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, q, k, v, causal, scale, label, heads=None):
    B, H = q.shape[:2]
    wo = wl = 0.0
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            o_ref, lse_ref = attention_rect(q[b, h], k[b, h], v[b, h], causal, scale)
            wo = max(wo, float(np.abs(o[b, h] - o_ref).max()))
            wl = max(wl, float(np.abs(lse[b, h] - lse_ref).max()))
    print(f"{label}: max|dO| {wo:.3e} max|dlse| {wl:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert wo <= 1e-2 and wl <= 1e-3
    assert wo <= o_bar(None, v) and wl <= LSE_BAR  # the dtype's own bar (bars.py)


CASES = [
    ("bf16", 128, 2, 4, 1, 1000, False), ("bf16", 128, 2, 4, 1, 1000, True), ("bf16", 128, 1, 8, 7, 777, True),
    ("bf16", 64, 2, 2, 32, 2000, True), ("f16", 128, 1, 4, 16, 4096, False), ("bf16", 128, 1, 2, 32, 32, True),
    ("bf16", 128, 3, 5, 5, 100, False), ("f16", 64, 1, 1, 3, 70000, True), ("bf16", 128, 1, 1, 1, 1, False),
    ("bf16", 256, 2, 4, 1, 1000, True), ("f16", 256, 1, 2, 32, 3000, False), ("bf16", 256, 1, 3, 7, 40000, True),
    # one query (the vector-ALU kernel): every head dimension and both types, ragged chunk ends
    ("f16", 64, 2, 3, 1, 5003, False), ("bf16", 64, 1, 2, 1, 77, True), ("f16", 128, 3, 3, 1, 20001, False),
    ("f16", 256, 1, 5, 1, 9999, True),
]


@pytest.mark.parametrize("dtype,d,B,H,Nq,Nk,causal", CASES)
def test_decode_sweep(dtype, d, B, H, Nq, Nk, causal):
    q, k, v = _inputs(B, H, Nq, Nk, d, dtype, seed=Nk + Nq)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q, k, v, causal, scale)
    _check(o, lse, q, k, v, causal, scale, f"{dtype} d{d} B{B} H{H} Nq{Nq} Nk{Nk} causal={causal}")


def test_decode_matches_forward_when_square_and_negative_scale():
    fa = _fa()
    q, k, v = _inputs(1, 3, 32, 32, 128, "bf16", seed=4)
    s = -float(np.float32(1 / np.sqrt(128)))
    o, lse = _run(q, k, v, True, s)
    _check(o, lse, q, k, v, True, s, "square, negative scale")
    of, lf = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=s)
    assert float(np.abs(of.float().cpu().numpy() - o).max()) <= 1e-2


@pytest.mark.parametrize("scale", [-0.0883883476, 0.0, 1.5])
def test_decode_single_query_scales(scale):
    # one query: negative scale (q sign-flipped), zero scale (uniform weights) and a large scale
    q, k, v = _inputs(2, 2, 1, 3000, 128, "bf16", seed=6)
    s = float(np.float32(scale))
    o, lse = _run(q, k, v, False, s)
    _check(o, lse, q, k, v, False, s, f"Nq1 scale={s}")


def test_decode_large_cache_sampled_heads():
    # B8 H32, one query against a 32768-key cache (the bench's decode workload); four heads checked
    q, k, v = _inputs(8, 32, 1, 32768, 128, "bf16", seed=8)
    scale = float(np.float32(1 / np.sqrt(128)))
    o, lse = _run(q, k, v, False, scale)
    rng = np.random.default_rng(1)
    heads = {divmod(int(x), 32) for x in rng.choice(256, size=4, replace=False)}
    _check(o, lse, q, k, v, False, scale, "B8 H32 Nq1 Nk32768", heads=heads)


@pytest.mark.parametrize("d,Nq,causal", [(64, 1, True), (128, 1, False), (256, 1, True), (64, 4, False),
                                         (128, 4, True), (256, 4, False)])
def test_decode_every_tail_length(d, Nq, causal):
    # key lengths Nq..Nq+69 (one chunk: every residue of the 32-key tile, twice) and a band where the keys
    # are split over several chunks with ragged ends; the vector kernel (Nq = 1) and the matrix kernel
    scale = float(np.float32(1 / np.sqrt(d)))
    for Nk in list(range(Nq, Nq + 70)) + list(range(4090, 4100)):
        q, k, v = _inputs(1, 2, Nq, Nk, d, "bf16", seed=3 * Nk + d + Nq)
        o, lse = _run(q, k, v, causal, scale)
        _check(o, lse, q, k, v, causal, scale, f"bf16 d{d} Nq{Nq} Nk{Nk} causal={causal}")

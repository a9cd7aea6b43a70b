"""GPU parity of fa_fwd_rect (Nq queries against Nk keys, causal queries starting at position q_start)
against the float64 oracle attention_rect, with the forward bar max|dO| <= 1e-2, max|dlse| <= 1e-3,
and the bitwise identities with fa_fwd that the kernel's row grouping implies."""

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


def _scale(d):
    return float(np.float32(1 / np.sqrt(d)))


def _inputs(dtype, d, B, H, Nq, Nk, seed):
    q = gen_qkv(B, H, Nq, d, dtype, seed=seed)[0]
    _, k, v = gen_qkv(B, H, Nk, d, dtype, seed=seed + 1)
    return q, k, v


CASES = [
    # dtype, d, B, H, Nq, Nk, q_start, causal
    ("bf16", 128, 2, 3, 200, 1000, 800, True),   # prefill chunk at the end of a cache
    ("f16", 64, 1, 2, 333, 1000, 300, True),     # middle range, ragged tiles on both sides
    ("bf16", 256, 1, 2, 130, 700, 257, True),
    ("f16", 128, 1, 2, 77, 500, 0, True),        # first range: sees a prefix of the keys only
    ("bf16", 128, 1, 3, 500, 129, 0, False),     # more queries than keys
    ("bf16", 64, 2, 2, 1, 50, 49, True),         # one query
    ("f16", 256, 1, 1, 64, 64, 0, True),
    ("bf16", 128, 1, 2, 40, 1, 0, False),        # one key
    ("f16", 64, 1, 1, 300, 4000, 1234, True),
    ("bf16", 256, 1, 1, 257, 2000, 0, False),
]


@pytest.mark.parametrize("dtype,d,B,H,Nq,Nk,q_start,causal", CASES)
def test_rect_matches_oracle(dtype, d, B, H, Nq, Nk, q_start, causal):
    fa = _fa()
    dev = torch.device("cuda")
    q, k, v = _inputs(dtype, d, B, H, Nq, Nk, seed=Nq + 7 * Nk + d)
    scale = _scale(d)
    print(f"rect {dtype} d{d} B{B} H{H} Nq{Nq} Nk{Nk} q_start{q_start} causal={causal}", flush=True)
    o, lse = fa.fwd_rect(q.to(dev), k.to(dev), v.to(dev), causal=causal, q_start=q_start, scale=scale)
    torch.cuda.synchronize()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    wo = wl = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, lse_ref = attention_rect(q[b, h], k[b, h], v[b, h], causal, scale, q_start=q_start)
            wo = max(wo, float(np.abs(o_np[b, h] - o_ref).max()))
            wl = max(wl, float(np.abs(lse_np[b, h] - lse_ref).max()))
    print(f"  max|dO| {wo:.3e} max|dlse| {wl:.3e}", flush=True)
    assert np.isfinite(o_np).all() and wo <= 1e-2 and wl <= 1e-3
    assert wo <= o_bar(dtype, v) and wl <= LSE_BAR  # the dtype's own bar (bars.py)


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("f16", 64, False), ("f16", 256, True)])
def test_rect_square_is_fa_fwd_bitwise(dtype, d, causal):
    fa = _fa()
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in gen_qkv(2, 2, 300, d, dtype, seed=d + 3))
    o1, l1 = fa.fwd(q, k, v, causal=causal)
    o2, l2 = fa.fwd_rect(q, k, v, causal=causal, q_start=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("f16", 256, True), ("bf16", 64, False)])
def test_rect_shards_reassemble_fa_fwd_bitwise(dtype, d, causal):
    # a sequence cut into query ranges at multiples of 128 rows with lengths that are multiples of 32
    # (or that end the sequence): each range against all keys gives fa_fwd's rows, bit for bit
    fa = _fa()
    dev = torch.device("cuda")
    N = 1000
    q, k, v = (t.to(dev) for t in gen_qkv(1, 3, N, d, dtype, seed=d + 11))
    o, lse = fa.fwd(q, k, v, causal=causal)
    for a, b in [(0, 256), (256, 640), (640, 1000), (128, 160)]:
        qs = q[:, :, a:b].contiguous()
        os_, ls = fa.fwd_rect(qs, k, v, causal=causal, q_start=a if causal else 0)
        torch.cuda.synchronize()
        assert torch.equal(os_, o[:, :, a:b]), f"o rows {a}:{b}"
        assert torch.equal(ls, lse[:, :, a:b]), f"lse rows {a}:{b}"


def test_rect_sharded_long_context_sampled_rows():
    # one GPU's share of a sequence-sharded causal forward at full size: fp16 B1 H8 d256, keys 16384,
    # queries 14336 .. 16383 (the last of eight ranges); sampled rows against the oracle
    fa = _fa()
    dev = torch.device("cuda")
    B, H, Nk, d, a = 1, 8, 16384, 256, 14336
    q, k, v = gen_qkv(B, H, Nk, d, "f16", seed=4)
    qs = q[:, :, a:].contiguous()
    scale = _scale(d)
    o, lse = fa.fwd_rect(qs.to(dev), k.to(dev), v.to(dev), causal=True, q_start=a, scale=scale)
    torch.cuda.synchronize()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 1023, 2046, 2047], rng.integers(0, Nk - a, 9)]))
    wo = wl = 0.0
    for h in (0, 5, 7):
        kh, vh = k[0, h].double().numpy(), v[0, h].double().numpy()  # exact upcast, once per head
        for r in rows:
            o_ref, lse_ref = attention_rect(qs[0, h, r:r + 1], kh, vh, True, scale, q_start=a + int(r))
            wo = max(wo, float(np.abs(o_np[0, h, r] - o_ref[0]).max()))
            wl = max(wl, float(abs(lse_np[0, h, r] - lse_ref[0])))
    print(f"rect f16 d256 Nq2048 Nk16384 q_start{a}: max|dO| {wo:.3e} max|dlse| {wl:.3e}", flush=True)
    assert np.isfinite(o_np).all() and wo <= 1e-2 and wl <= 1e-3
    assert wo <= o_bar("f16", v) and wl <= LSE_BAR


@pytest.mark.parametrize("dtype,d,a", [("bf16", 128, 1000), ("f16", 256, 1000), ("bf16", 128, 1056)])
def test_rect_unaligned_start_every_dispatch_round(dtype, d, a):
    # causal query rows starting at a position that is not a multiple of 32 (1000: both key orders would
    # leave rows without a key in their first tile, so the grid walks upward), or a multiple of 32 but not
    # of the 64-key tile (1056: odd dispatch rounds walk downward), on a grid of two dispatch rounds (B1
    # H16, 8192 query rows: 1024 workgroups of 128 rows at d = 128, 512 of 256 rows at d = 256); every
    # output finite, sampled rows of the first and last heads against the oracle
    fa = _fa()
    dev = torch.device("cuda")
    B, H, Nq = 1, 16, 8192
    Nk = a + Nq
    q, k, v = _inputs(dtype, d, B, H, Nq, Nk, seed=d + 21)
    scale = _scale(d)
    o, lse = fa.fwd_rect(q.to(dev), k.to(dev), v.to(dev), causal=True, q_start=a, scale=scale)
    bad = int((~torch.isfinite(o)).any(dim=-1).sum()) + int((~torch.isfinite(lse)).sum())
    assert bad == 0, f"{bad} non-finite output rows or lse values"
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(d)
    tile = 128 if d <= 128 else 256
    rows = np.unique(np.concatenate([np.arange(0, Nq, tile), np.arange(31, Nq, tile), rng.integers(0, Nq, 8)]))
    wo = wl = 0.0
    for h in (0, H - 1):
        kh, vh = k[0, h].double().numpy(), v[0, h].double().numpy()
        for r in rows:
            o_ref, lse_ref = attention_rect(q[0, h, r:r + 1], kh, vh, True, scale, q_start=a + int(r))
            wo = max(wo, float(np.abs(o_np[0, h, r] - o_ref[0]).max()))
            wl = max(wl, float(abs(lse_np[0, h, r] - lse_ref[0])))
    print(f"rect {dtype} d{d} B{B} H{H} Nq{Nq} Nk{Nk} q_start{a}: max|dO| {wo:.3e} max|dlse| {wl:.3e}", flush=True)
    assert wo <= 1e-2 and wl <= 1e-3
    assert wo <= o_bar(dtype, v) and wl <= LSE_BAR


def test_rect_rejects_bad_start():
    fa = _fa()
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in gen_qkv(1, 1, 64, 64, "bf16", seed=9))
    with pytest.raises(fa.FaError):
        fa.fwd_rect(q, k[:, :, :32].contiguous(), v[:, :, :32].contiguous(), causal=True, q_start=0)
    with pytest.raises(ValueError):
        fa.fwd_rect(q, k, v, out=torch.empty((1, 1, 63, 64), dtype=q.dtype, device=dev))

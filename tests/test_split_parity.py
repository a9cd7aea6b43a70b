"""GPU parity of fa_fwd_split (each query tile's keys split into shares, partial results merged)
against the float64 oracle attention_rect, with the forward bar max|dO| <= 1e-2, max|dlse| <= 1e-3;
nsplit = 1 reproduces fa_fwd_rect bit for bit (one share is the unsplit kernel, and the merge of one
partial is exact)."""

import numpy as np
import pytest
import torch

from bars import LSE_BAR, o_bar
from oracle import attention_rect
from synth import gen_qkv

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


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
    # dtype, d, B, H, Nq, Nk, q_start, causal, nsplit
    ("bf16", 128, 1, 2, 300, 1000, 700, True, 3),    # prefill chunk at the end of a cache
    ("f16", 64, 1, 2, 200, 200, 0, True, 4),         # square causal: early rows see nothing of late shares
    ("bf16", 256, 1, 2, 129, 777, 0, False, 5),      # ragged query and key tiles
    ("f16", 128, 1, 1, 64, 5000, 0, False, 16),      # few queries, long keys
    ("bf16", 64, 2, 1, 1, 300, 299, True, 7),        # more shares than key tiles: empty shares
    ("f16", 256, 1, 1, 256, 4096, 3840, True, 8),
    ("bf16", 128, 2, 2, 500, 129, 0, False, 2),      # more queries than keys
    ("f16", 64, 1, 1, 333, 4000, 1234, True, 6),     # middle range of a sequence
    ("bf16", 256, 1, 2, 300, 1000, 700, True, 3),    # d = 256 (in-order pipeline), ragged causal range
    ("f16", 128, 1, 2, 1000, 1000, 0, True, 64),     # the largest share count: most shares empty for early rows
]


@pytest.mark.parametrize("dtype,d,B,H,Nq,Nk,q_start,causal,nsplit", CASES)
def test_split_matches_oracle(dtype, d, B, H, Nq, Nk, q_start, causal, nsplit):
    fa = _fa()
    q, k, v = _inputs(dtype, d, B, H, Nq, Nk, seed=Nq * 3 + Nk + nsplit)
    dev = torch.device("cuda")
    o, lse = fa.fwd_split(q.to(dev), k.to(dev), v.to(dev), nsplit=nsplit, causal=causal, q_start=q_start,
                          scale=_scale(d))
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = attention_rect(q[b, h], k[b, h], v[b, h], causal, _scale(d), q_start)
            worst_o = max(worst_o, float(np.abs(o[b, h] - o_ref).max()))
            worst_l = max(worst_l, float(np.abs(lse[b, h] - l_ref).max()))
    print(f"split {dtype} d{d} B{B} H{H} Nq{Nq} Nk{Nk} q_start={q_start} causal={causal} nsplit={nsplit}: "
          f"max|dO|={worst_o:.3e} max|dlse|={worst_l:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert worst_o <= TOL_O and worst_l <= TOL_LSE
    assert worst_o <= o_bar(dtype, v) and worst_l <= LSE_BAR  # the dtype's own bar (bars.py)


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("f16", 64, False), ("f16", 256, True)])
def test_one_share_is_rect_bitwise(dtype, d, causal):
    fa = _fa()
    Nq, Nk = 300, 900
    q, k, v = (t.cuda() for t in _inputs(dtype, d, 1, 2, Nq, Nk, seed=41 + d))
    qs = Nk - Nq if causal else 0
    o1, l1 = fa.fwd_rect(q, k, v, causal=causal, q_start=qs)
    o2, l2 = fa.fwd_split(q, k, v, nsplit=1, causal=causal, q_start=qs)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_split_deterministic_and_workspace_reuse():
    fa = _fa()
    q, k, v = (t.cuda() for t in _inputs("bf16", 128, 2, 2, 400, 3000, seed=77))
    ws = torch.empty(fa.split_workspace_bytes(2, 2, 400, 128, 6), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.fwd_split(q, k, v, nsplit=6, causal=True, q_start=2600, workspace=ws)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = fa.fwd_split(q, k, v, nsplit=6, causal=True, q_start=2600, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_sequence_share_full_size_sampled_rows():
    # the last of eight query ranges of the fp16 B1 H8 N16384 d256 causal workload against its keys, in
    # the launch configuration of the shard bench (4 shares), checked on sampled rows
    fa = _fa()
    N, G, d, H = 16384, 8, 256, 8
    nq = N // G
    q0 = N - nq
    q, k, v = gen_qkv(1, H, N, d, "f16", seed=4)
    qd = q[:, :, q0:].contiguous().cuda()
    kd, vd = k.cuda(), v.cuda()
    o, lse = fa.fwd_split(qd, kd, vd, nsplit=4, causal=True, q_start=q0, scale=_scale(d))
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rng = np.random.default_rng(5)
    worst_o = worst_l = 0.0
    for h in (0, 5):
        for r in np.unique(np.concatenate([[0, 1, nq - 1], rng.integers(0, nq, 6)])):
            o_ref, l_ref = attention_rect(q[0, h, q0 + r:q0 + r + 1], k[0, h], v[0, h], True, _scale(d), q0 + r)
            worst_o = max(worst_o, float(np.abs(o[0, h, r] - o_ref[0]).max()))
            worst_l = max(worst_l, abs(float(lse[0, h, r] - l_ref[0])))
    print(f"split fp16 share rows {q0}..{N - 1} of N{N} d{d}: sampled max|dO|={worst_o:.3e} "
          f"max|dlse|={worst_l:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert worst_o <= TOL_O and worst_l <= TOL_LSE
    assert worst_o <= o_bar("f16", v) and worst_l <= LSE_BAR

"""The library's launches under HIP graph capture (torch.cuda.CUDAGraph): the entry points allocate
nothing and issue only kernels on the caller's stream, so a captured forward, backward, decode or split forward replays
to the same bits as the eager call.  Each graph is replayed several times with eager work and
synchronisation in between, and every replay is compared with the eager result."""

import numpy as np
import pytest
import torch

from synth import gen_qkv

pytestmark = pytest.mark.gpu


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


def _capture(fn):
    """Warm up on a side stream (as torch requires before capture), then capture fn into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_replay_bitwise(causal):
    fa = _fa()
    dev = torch.device("cuda")
    B, H, N, d = 2, 3, 333, 128
    q, k, v = (t.to(dev) for t in gen_qkv(B, H, N, d, "bf16", seed=41))
    g_out = gen_qkv(B, H, N, d, "bf16", seed=42)[0].to(dev)
    scale = float(np.float32(1 / np.sqrt(d)))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)

    def step():
        fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, g_out, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    graph = _capture(step)
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between replays; any stale value would show
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"


def test_decode_replay_bitwise():
    fa = _fa()
    dev = torch.device("cuda")
    B, H, Nq, Nk, d = 2, 4, 1, 5000, 128
    qf, k, v = (t.to(dev) for t in gen_qkv(B, H, Nk, d, "bf16", seed=43))
    q = qf[:, :, Nk - Nq:, :].contiguous()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(B, H, Nq, Nk, d), dtype=torch.uint8, device=dev)

    def step():
        fa.fwd_decode(q, k, v, causal=True, out=o, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    graph = _capture(step)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"decode replay {rep} differs"


def test_split_replay_bitwise():
    # key shares and their merge (two launches, partials in the caller's workspace); the workspace is
    # overwritten between replays: every share writes all of its partial rows, empty ones included
    fa = _fa()
    dev = torch.device("cuda")
    B, H, Nq, Nk, d, ns = 1, 3, 300, 2000, 128, 5
    q = gen_qkv(B, H, Nq, d, "bf16", seed=44)[0].to(dev)
    _, k, v = (t.to(dev) for t in gen_qkv(B, H, Nk, d, "bf16", seed=45))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.split_workspace_bytes(B, H, Nq, d, ns), dtype=torch.uint8, device=dev)

    def step():
        fa.fwd_split(q, k, v, nsplit=ns, causal=True, q_start=Nk - Nq, out=o, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    graph = _capture(step)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"split replay {rep} differs"


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_prep_and_forward_replay_bitwise(causal):
    # the e4m3 path: three preparation launches (Q and K rotated) and the e4m3 forward, all into the
    # caller's buffers; codes, scales, output and lse overwritten between replays
    from synth import gen_signs

    fa = _fa()
    dev = torch.device("cuda")
    B, H, N, d = 2, 2, 300, 128
    q, k, v = (t.to(dev) for t in gen_qkv(B, H, N, d, "bf16", seed=46, outlier_frac=0.001, outlier_mult=20.0))
    signs = gen_signs(d, seed=d)
    nblk = -(-N // 64)
    codes = [torch.empty(q.shape, dtype=torch.float8_e4m3fn, device=dev) for _ in range(3)]
    scales = [torch.empty((B, H, nblk), dtype=torch.float32, device=dev) for _ in range(3)]
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    def step():
        for x, sg, c, s in zip((q, k, v), (signs, signs, None), codes, scales):
            fa.fp8_prep(x, sg, 64, out=c, scales=s)
        fa.fwd(*codes, causal=causal, fp8_scales=tuple(scales), out=o, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*codes, *scales, o, lse)]
    graph = _capture(step)
    for rep in range(3):
        for c in codes:
            c.view(torch.uint8).fill_(0x7F)  # e4m3 NaN codes
        for t in (*scales, o, lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (*codes, *scales, o, lse)
        for i, (g, w) in enumerate(zip(got, ref)):
            same = torch.equal(g.view(torch.uint8), w.view(torch.uint8)) if g.dtype == torch.float8_e4m3fn else torch.equal(g, w)
            assert same, f"fp8 replay {rep}: output {i} differs from the eager result"

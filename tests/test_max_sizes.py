"""The largest shapes the C ABI accepts, checked against the float64 oracle on sampled rows and heads.

* The longest sequence: N = 2^21 - 1 (the entry points reject N >= 2^21, which keeps every in-head
  byte offset the kernels form below 2^31), causal, with a ragged last tile.  Offsets inside a head
  reach 2^30 bytes at d = 256.
* More than 2^31 elements per tensor: 131 200 heads of 128 x 128, so head offsets pass 2^32 bytes;
  forward and backward, sampled heads at the start, the middle and the very end.

Inputs are drawn on the device (synth.gen_qkv_device); the sampled heads are copied back to the host
for the oracle.  Tolerances are those of the other parity tests: max|dO| <= 1e-2, max|dlse| <= 1e-3,
and max|d - d_ref| <= 5 * 2^-8 max|d_ref| per gradient (bfloat16).
"""

import math

import numpy as np
import pytest
import torch

from bars import LSE_BAR, o_bar
from oracle import attention_bwd_rows, attention_rows
from synth import gen_qkv_device

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, REL = 1e-2, 1e-3, 5 * 2.0 ** -8  # the backward parity bar for bfloat16 (5 unit roundoffs)
N_MAX = (1 << 21) - 1


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f16", 256)])
def test_longest_sequence_causal(dtype, d):
    fa = _fa()
    dev = torch.device("cuda")
    print(f"longest sequence: {dtype} d{d} N{N_MAX} causal", flush=True)
    q, k, v = gen_qkv_device(1, 1, N_MAX, d, dtype, seed=d + 7, device=dev)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(d)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, N_MAX // 2, N_MAX - 64, N_MAX - 2, N_MAX - 1],
                                     rng.integers(0, N_MAX, 8)]))
    ri = torch.from_numpy(rows).to(dev)
    o_got = o[0, 0].index_select(0, ri).float().cpu().numpy()
    l_got = lse[0, 0].index_select(0, ri).cpu().numpy()
    assert np.isfinite(o_got).all() and np.isfinite(l_got).all()
    qh, kh, vh = (t[0, 0].cpu() for t in (q, k, v))
    del q, k, v, o, lse
    o_ref, l_ref = attention_rows(qh, kh, vh, rows, True, scale)
    do = float(np.abs(o_got - o_ref).max())
    dl = float(np.abs(l_got - l_ref).max())
    print(f"  {len(rows)} rows: max|dO|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert do <= TOL_O and dl <= TOL_LSE
    assert do <= o_bar(dtype, vh) and dl <= LSE_BAR  # the dtype's own bar (bars.py)


def test_past_2_31_elements_forward_and_backward():
    fa = _fa()
    dev = torch.device("cuda")
    B, H, N, d = 1, 131200, 128, 128
    assert B * H * N * d > 2 ** 31
    print(f"many heads: bf16 B{B} H{H} N{N} d{d} causal", flush=True)
    q, k, v, dout = gen_qkv_device(B, H, N, d, "bf16", seed=5, device=dev, count=4)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dout, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    heads = sorted({0, 1, H // 2, H - 2, H - 1, *rng.integers(0, H, 3).tolist()})
    rows = np.arange(N)
    for h in heads:
        qh, kh, vh, gh = (t[0, h].cpu() for t in (q, k, v, dout))
        o_ref, l_ref = attention_rows(qh, kh, vh, rows, True, scale)
        do_ = float(np.abs(o[0, h].float().cpu().numpy() - o_ref).max())
        dl = float(np.abs(lse[0, h].cpu().numpy() - l_ref).max())
        line = f"  head {h}: max|dO|={do_:.3e} max|dlse|={dl:.3e}"
        assert do_ <= TOL_O and dl <= TOL_LSE, line
        assert do_ <= o_bar("bf16", vh) and dl <= LSE_BAR, line
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), attention_bwd_rows(qh, kh, vh, gh, True, scale)):
            g = got[0, h].float().cpu().numpy()
            err, top = float(np.abs(g - ref).max()), float(np.abs(ref).max())
            line += f" {name} {err / top:.2e}"
            assert np.isfinite(g).all() and err <= REL * top + 1e-6, line
        print(line, flush=True)

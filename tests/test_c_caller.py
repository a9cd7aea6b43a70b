"""The C ABI called from a plain C99 program (tests/c_caller/fa_c_forward.c: HIP runtime allocations,
fa_fwd on the null stream, no Python or PyTorch in the process), on the GPU: its output matches the
float64 oracle at the forward bars and is bitwise the Python binding's output for the same inputs (the
same library entry point and launch)."""
import math
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

from bars import LSE_BAR, o_bar
from oracle import attention_ref
from synth import gen_qkv

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_caller", "fa_c_forward")
CODES = {"f32": (0, torch.float32), "f16": (1, torch.float16), "bf16": (2, torch.bfloat16)}


@pytest.mark.parametrize("dtype,d,B,H,N,causal", [("bf16", 128, 2, 3, 333, True), ("f16", 256, 1, 2, 700, False),
                                                  ("f16", 64, 2, 2, 129, True), ("f32", 128, 1, 2, 150, False)])
def test_c_program_matches_oracle_and_binding(dtype, d, B, H, N, causal, tmp_path):
    assert os.path.exists(EXE), "tests/c_caller/fa_c_forward is not built: run __graft_entry__.build()"
    import exact_tiled_attention_22_amd as fa

    code, tdt = CODES[dtype]
    q, k, v = gen_qkv(B, H, N, d, dtype, seed=N + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<6if", B, H, N, d, int(causal), code, scale))
        for t in (q, k, v):
            f.write(t.contiguous().view(torch.uint8).numpy().tobytes())
    print(f"C caller: {dtype} d{d} B{B} H{H} N{N} causal={causal}", flush=True)
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, dtype=np.uint8)
    nbytes = B * H * N * d * tdt.itemsize
    assert raw.size == nbytes + B * H * N * 4
    o_c = torch.from_numpy(raw[:nbytes].copy()).view(tdt).reshape(B, H, N, d)
    lse_c = torch.from_numpy(raw[nbytes:].copy()).view(torch.float32).reshape(B, H, N)
    # the Python binding on the same inputs: the same entry point, hence the same bits
    dev = torch.device("cuda")
    o_p, lse_p = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_c.view(torch.uint8), o_p.cpu().contiguous().view(torch.uint8))
    assert torch.equal(lse_c, lse_p.cpu())
    o_ref, lse_ref = attention_ref(q, k, v, causal, scale)
    do = float(np.abs(o_c.float().numpy() - o_ref).max())
    dl = float(np.abs(lse_c.numpy() - lse_ref).max())
    print(f"  max|dO|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert do <= 1e-2 and do <= o_bar(dtype, v) and dl <= 1e-3 and dl <= LSE_BAR


def test_c_program_reports_a_rejected_request(tmp_path):
    assert os.path.exists(EXE), "tests/c_caller/fa_c_forward is not built: run __graft_entry__.build()"
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    B, H, N, d = 1, 1, 8, 96  # head dimension 96 is not supported: FA_ERR_UNSUPPORTED before any launch
    with open(src, "wb") as f:
        f.write(struct.pack("<6if", B, H, N, d, 0, 2, 0.1))
        f.write(bytes(3 * B * H * N * d * 2))
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "FA_ERR_UNSUPPORTED" in r.stderr

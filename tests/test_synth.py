"""The seeded generator: determinism, distribution and the outlier recipe (CPU only)."""

import numpy as np
import torch

from synth import WORKLOADS, gen_qkv, gen_signs


def test_same_seed_same_bits_and_streams_differ():
    a = gen_qkv(1, 2, 33, 16, "bf16", seed=5)
    b = gen_qkv(1, 2, 33, 16, "bf16", seed=5)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.is_contiguous()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a[0], a[1]) and not torch.equal(a[1], a[2])
    c = gen_qkv(1, 2, 33, 16, "bf16", seed=6)
    assert not torch.equal(a[0], c[0])


def test_values_are_standard_normal_rounded_to_dtype():
    q, _, _ = gen_qkv(1, 4, 512, 64, "f16", seed=1)
    x = q.float().numpy().astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    # the stored tensor holds fp16 values exactly
    assert torch.equal(q.float().half(), q)


def test_outlier_count_and_factor():
    B, H, N, d = 1, 2, 256, 64
    plain = gen_qkv(B, H, N, d, "f32", seed=9)
    out = gen_qkv(B, H, N, d, "f32", seed=9, outlier_frac=0.001, outlier_mult=20.0)
    want = int(round(0.001 * B * H * N * d))
    for p, o in zip(plain, out):
        changed = (p != o).reshape(-1)
        assert int(changed.sum()) == want
        np.testing.assert_allclose(o.reshape(-1)[changed].numpy(), 20.0 * p.reshape(-1)[changed].numpy(),
                                   rtol=1e-6)


def test_signs_and_config_table():
    s = gen_signs(128, 5)
    assert s.dtype == np.int8 and set(np.unique(s)) <= {-1, 1} and len(s) == 128
    assert [c.dtype for c in WORKLOADS.values()] == ["f32", "bf16", "bf16", "f16", "fp8"]
    assert WORKLOADS[2].flops == 4.0 * 16 * 16 * 1024 * 1024 * 128
    assert WORKLOADS[3].flops == 2.0 * 2 * 16 * 8192 * 8192 * 128
    assert WORKLOADS[4].scale == 0.0625 and WORKLOADS[1].scale == 0.125

"""GPU parity of the fp8 preparation kernel (bitwise) and the fp8 forward (RMSE) against the oracle."""

import numpy as np
import pytest
import torch

from oracle import attention_ref, fp8_attention_ref, fp8_prep_ref
from synth import CONFIGS, gen_fp8_workload, gen_qkv, gen_signs

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

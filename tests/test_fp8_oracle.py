"""Pins of the oracle's fp8 pieces (CPU only): e4m3 codec, Walsh-Hadamard transform, block absmax
quantisation.  Independent references: torch.float8_e4m3fn conversions, scipy.linalg.hadamard,
code values fixed by the OCP 8-bit floating point specification, and error bounds of the format.
"""

import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import (
    attention_ref,
    dequantize_blocks,
    e4m3_decode,
    e4m3_encode,
    fp8_attention_ref,
    fp8_prep_ref,
    fwht_f32,
)


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2  # 0x7F and 0xFF only
    np.testing.assert_array_equal(ours[~nan], theirs[~nan])


def test_known_codes_from_the_format_definition():
    # OCP e4m3fn: 1.0 = 0 0111 000, 448 = 0 1111 110, 2^-6 = 0 0001 000, 2^-9 = 0 0000 001
    vals = [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, -1.0, 0.0, -0.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 460.0, 1e6]
    want = [0x38, 0x7E, 0x08, 0x01, 0xB8, 0x00, 0x80, 0x00, 0x01, 0x7E, 0x7E]
    assert list(e4m3_encode(np.array(vals))) == want


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_round_to_nearest_even_matches_torch():
    # every representable value, every midpoint between neighbours, and random values below 464
    pos = np.unique(e4m3_decode(np.arange(0, 127, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    rnd = np.random.default_rng(5).uniform(-463.9, 463.9, 20000)
    x = np.concatenate([pos, -pos, mids, -mids, rnd, [448.0 + 15.99, -(448.0 + 15.99)]]).astype(np.float32)
    ours = e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_equals_sylvester_matrix(d):
    # small integers: every float32 butterfly is exact, so the result must equal y @ H_d exactly
    y = np.random.default_rng(d).integers(-8, 9, size=(5, d)).astype(np.float32)
    hd = scipy.linalg.hadamard(d)
    np.testing.assert_array_equal(fwht_f32(y).astype(np.float64), y.astype(np.float64) @ hd)
    np.testing.assert_array_equal(hd @ hd.T, d * np.eye(d))


def test_fwht_float32_error_bound():
    d = 128
    y = np.random.default_rng(3).standard_normal((64, d)).astype(np.float32)
    exact = y.astype(np.float64) @ scipy.linalg.hadamard(d)
    bound = math.log2(d) * 2.0 ** -24 * (np.abs(y).astype(np.float64) @ np.abs(scipy.linalg.hadamard(d)))
    assert (np.abs(fwht_f32(y) - exact) <= bound + 1e-30).all()


def _rows(shape, seed, outliers=0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    if outliers:
        idx = np.random.default_rng(seed + 1).choice(x.size, outliers, replace=False)
        x.reshape(-1)[idx] *= 20
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("rotate", [False, True])
def test_prep_quantisation_error_and_amax(rotate):
    BH, N, d, block = 3, 200, 128, 64  # 200 = 3 full blocks + a partial one of 8 rows
    x = _rows((BH, N, d), 7, outliers=40)
    signs = np.where(np.random.default_rng(8).integers(0, 2, d) == 1, 1, -1).astype(np.int8) if rotate else None
    codes, scales = fp8_prep_ref(x, signs, block)
    assert codes.shape == x.shape and codes.dtype == np.uint8
    assert scales.shape == (BH, 4) and scales.dtype == np.float32
    ref = x.astype(np.float64)
    if rotate:
        r = np.diag(signs.astype(np.float64)) @ scipy.linalg.hadamard(d) / math.sqrt(d)
        ref = ref @ r
    deq = dequantize_blocks(codes, scales, block)
    for b in range(4):
        sl = slice(64 * b, min(N, 64 * (b + 1)))
        amax = np.abs(ref[:, sl]).max(axis=(1, 2))
        # scale = amax / 448 (up to the float32 rounding of the rotation)
        np.testing.assert_allclose(scales[:, b], amax / 448.0, rtol=1e-5)
        # the largest element of each block lands on code +-448
        blk = codes[:, sl] & 0x7F
        assert (blk.reshape(BH, -1).max(axis=1) == 0x7E).all()
        # e4m3 error: half a unit in the last place of 3 mantissa bits, or half the subnormal step
        err = np.abs(deq[:, sl] - ref[:, sl])
        sc = scales[:, b][:, None, None].astype(np.float64)
        bound = np.maximum(np.abs(ref[:, sl]) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-5) + sc * 1e-5
        assert (err <= bound).all()


def test_prep_zero_block_and_sign_handling():
    x = np.zeros((1, 70, 64), dtype=np.float32)
    x[0, 64:] = -1.0  # second (partial) block: all -1
    codes, scales = fp8_prep_ref(x, None, 64)
    assert scales[0, 0] == 1.0 and (codes[0, :64] == 0).all()
    assert scales[0, 1] == np.float32(1.0 / 448.0) and (codes[0, 64:] == 0xFE).all()  # -448


def test_rotation_preserves_scores_before_quantisation():
    N, d = 16, 64
    q, k = _rows((1, N, d), 11), _rows((1, N, d), 12)
    s = np.where(np.random.default_rng(13).integers(0, 2, d) == 1, 1, -1).astype(np.int8)
    rs = np.float32(1.0 / np.sqrt(d))
    qr = fwht_f32(q * s) * rs
    kr = fwht_f32(k * s) * rs
    np.testing.assert_allclose(qr[0].astype(np.float64) @ kr[0].T.astype(np.float64),
                               q[0].astype(np.float64) @ k[0].T.astype(np.float64), atol=2e-5)


def test_fp8_attention_ref_on_exact_codes_is_plain_attention():
    # inputs that are exactly code * scale dequantise to themselves
    N, d, block = 96, 64, 64
    rng = np.random.default_rng(17)
    codes = [rng.integers(0, 0x7E, size=(1, N, d)).astype(np.uint8) for _ in range(3)]
    scales = [np.full((1, 2), 0.01 * (i + 1), dtype=np.float32) for i in range(3)]
    o, lse = fp8_attention_ref(codes[0], scales[0], codes[1], scales[1], codes[2], scales[2],
                               block, False, 0.125)
    deq = [e4m3_decode(c) * np.float64(s[0, 0]) for c, s in zip(codes, scales)]
    o2, lse2 = attention_ref(*deq, False, 0.125)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)

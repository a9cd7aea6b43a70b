"""Pins of the float64 attention oracle against things other than itself (CPU only).

Each test names the plausible mistake it would catch.  The pages print no worked example, so the
pins are: brute force with math.fsum on tiny inputs, torch's float64 scaled_dot_product_attention
and scipy's logsumexp (independent library routines), closed forms and invariances of the softmax
definition (FlashAttention 2 + 3 — speicherbewusste Attention-Kernels, "Kernpunkte").
"""

import math

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

from oracle import attention_ref, attention_rows


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _brute(q, k, v, causal, scale):
    """Direct evaluation with math.exp / math.fsum, no max subtraction, pure Python loops."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        w = {j: math.exp(scale * math.fsum(q[i][t] * k[j][t] for t in range(d))) for j in keys}
        z = math.fsum(w.values())
        for c in range(dv):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in keys) / z
        lse[i] = math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("n,d", [(1, 1), (2, 3), (3, 2), (5, 4), (8, 8), (7, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(n, d, causal):
    # catches: any formula error (dropped scale, wrong mask side, swapped K/V, lse without max)
    seed = 1000 * n + 10 * d + int(causal)
    q, k, v = _rand((n, d), seed), _rand((n, d), seed + 1), _rand((n, d), seed + 2)
    scale = 0.7 / math.sqrt(d)
    o_ref, lse_ref = _brute(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    o, lse = attention_ref(q[None, None], k[None, None], v[None, None], causal, scale)
    np.testing.assert_allclose(o[0, 0], o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    # independent library implementation; catches mask off-by-one, transposed operands, scale errors
    B, H, N, d = 2, 3, 37, 16
    q, k, v = (_rand((B, H, N, d), s) for s in (1, 2, 3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_ref(q, k, v, causal, scale, row_chunk=8)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o_t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=0, atol=1e-12)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_prefix_mean(causal):
    # closed form: Q = 0 -> all scores 0 -> uniform weights; catches wrong normaliser / mask
    N, d = 29, 8
    v = _rand((N, d), 7)
    q = np.zeros((N, d))
    k = _rand((N, d), 8)
    o, lse = attention_ref(q[None], k[None], v[None], causal, 0.3)
    for i in range(N):
        cnt = i + 1 if causal else N
        np.testing.assert_allclose(o[0, i], v[:cnt].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, i] - math.log(cnt)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_that_constant(causal):
    # softmax weights sum to one: V[j] = c for all j -> O[i] = c; catches missing 1/l
    N, d = 41, 6
    q, k = _rand((N, d), 11, 3.0), _rand((N, d), 12, 3.0)
    c = _rand((d,), 13)
    v = np.tile(c, (N, 1))
    o, _ = attention_ref(q[None], k[None], v[None], causal, 1.0)
    np.testing.assert_allclose(o[0], np.tile(c, (N, 1)), rtol=0, atol=1e-13)


def test_causal_row_zero_is_first_value():
    # causal row 0 sees only key 0: O[0] = V[0], lse[0] = scale * q0.k0; catches a mask off by one
    N, d = 16, 8
    q, k, v = _rand((N, d), 21), _rand((N, d), 22), _rand((N, d), 23)
    scale = 0.125
    o, lse = attention_ref(q[None], k[None], v[None], True, scale)
    np.testing.assert_array_equal(o[0, 0], v[0])
    assert abs(lse[0, 0] - scale * float(q[0] @ k[0])) < 1e-14


def test_two_keys_is_logistic():
    # N = 2 non-causal: weight of key 0 is the logistic function of s0 - s1
    d = 4
    q, k, v = _rand((2, d), 31), _rand((2, d), 32), _rand((2, d), 33)
    scale = 0.5
    o, lse = attention_ref(q[None], k[None], v[None], False, scale)
    for i in range(2):
        s0, s1 = scale * q[i] @ k[0], scale * q[i] @ k[1]
        w0 = scipy.special.expit(s0 - s1)
        np.testing.assert_allclose(o[0, i], w0 * v[0] + (1 - w0) * v[1], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, i], np.logaddexp(s0, s1), rtol=0, atol=1e-14)


def test_identity_values_expose_probabilities():
    # V = I: O is the probability matrix itself; rows are non-negative and sum to one, and
    # P_ij = exp(s_ij - lse_i) ties O to lse; catches a wrong lse or a missing normalisation
    N = 24
    q, k = _rand((N, N), 41, 2.0), _rand((N, N), 42, 2.0)
    scale = 0.2
    for causal in (False, True):
        o, lse = attention_ref(q[None], k[None], np.eye(N)[None], causal, scale)
        p = o[0]
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        s = scale * q @ k.T
        expect = np.exp(s - lse[0][:, None])
        if causal:
            expect = np.tril(expect)
        np.testing.assert_allclose(p, expect, rtol=0, atol=1e-13)


def test_joint_key_value_permutation_and_query_permutation():
    # non-causal attention is a set function of the (key, value) pairs; query rows are independent
    N, d = 33, 8
    q, k, v = _rand((N, d), 51), _rand((N, d), 52), _rand((N, d), 53)
    perm = np.random.default_rng(54).permutation(N)
    o, lse = attention_ref(q[None], k[None], v[None], False, 0.4)
    o2, lse2 = attention_ref(q[None], k[perm][None], v[perm][None], False, 0.4)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    o3, lse3 = attention_ref(q[perm][None], k[None], v[None], False, 0.4)
    np.testing.assert_allclose(o3[0], o[0][perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse3[0], lse[0][perm], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_per_row_score_shift(causal):
    # adding the same vector w to every key adds scale*q_i.w to row i's scores: O unchanged,
    # lse shifted by exactly that amount; catches a wrong max subtraction or lse offset
    N, d = 31, 8
    q, k, v = _rand((N, d), 61), _rand((N, d), 62), _rand((N, d), 63)
    w = _rand((d,), 64, 2.0)
    scale = 0.35
    o, lse = attention_ref(q[None], k[None], v[None], causal, scale)
    o2, lse2 = attention_ref(q[None], (k + w)[None], v[None], causal, scale)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2[0], lse[0] + scale * (q @ w), rtol=0, atol=1e-12)


def test_orthogonal_rotation_of_queries_and_keys():
    # (Q R)(K R)^T = Q K^T for the orthogonal R = D_s H_d / sqrt(d) used by the fp8 path
    N, d = 20, 16
    q, k, v = _rand((N, d), 71), _rand((N, d), 72), _rand((N, d), 73)
    s = np.where(np.random.default_rng(74).integers(0, 2, d) == 1, 1.0, -1.0)
    r = np.diag(s) @ scipy.linalg.hadamard(d) / math.sqrt(d)
    np.testing.assert_allclose(r @ r.T, np.eye(d), atol=1e-14)
    o, lse = attention_ref(q[None], k[None], v[None], True, 0.25)
    o2, lse2 = attention_ref((q @ r)[None], (k @ r)[None], v[None], True, 0.25)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_rows_helper_equals_full_and_chunking_is_invisible():
    N, d = 70, 8
    q, k, v = _rand((N, d), 81), _rand((N, d), 82), _rand((N, d), 83)
    for causal in (False, True):
        o_full, lse_full = attention_ref(q[None], k[None], v[None], causal, 0.3, row_chunk=1024)
        o_ch, lse_ch = attention_ref(q[None], k[None], v[None], causal, 0.3, row_chunk=9)
        np.testing.assert_array_equal(o_full, o_ch)
        rows = np.array([0, 5, 69, 33])
        o_r, lse_r = attention_rows(q, k, v, rows, causal, 0.3)
        np.testing.assert_array_equal(o_r, o_full[0][rows])
        np.testing.assert_array_equal(lse_r, lse_full[0][rows])


def test_accepts_torch_low_precision_tensors_exactly():
    # the oracle upcasts bf16/fp16 tensors exactly (no second rounding)
    x = torch.randn(1, 1, 8, 4).to(torch.bfloat16)
    o, _ = attention_ref(x, x, x, False, 1.0)
    o2, _ = attention_ref(x.float().numpy().astype(np.float64), x.float().numpy(), x.float().numpy(),
                          False, 1.0)
    np.testing.assert_array_equal(o, o2)

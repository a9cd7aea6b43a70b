"""Pins of the rectangular (decode-shape) oracle — CPU only."""

import math

import numpy as np
import pytest
import torch

from oracle import attention_rect, attention_rows


def test_rect_equals_square_when_nq_equals_nk():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((40, 16)) for _ in range(3))
    for causal in (False, True):
        o, lse = attention_rect(q, k, v, causal, 0.3)
        o2, lse2 = attention_rows(q, k, v, np.arange(40), causal, 0.3)
        np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_rect_matches_torch_with_explicit_mask(causal):
    rng = np.random.default_rng(2)
    nq, nk, d = 5, 77, 32
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    mask = None
    if causal:
        mask = torch.tensor(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + (nk - nq))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                                           attn_mask=mask, scale=0.2)
    o, _ = attention_rect(q, k, v, causal, 0.2)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rect_brute_force_single_query():
    # one query: the last key position of a causal sequence sees every key
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((1, 3)), rng.standard_normal((6, 3)), rng.standard_normal((6, 3))
    s = [0.5 * math.fsum(q[0, t] * k[j, t] for t in range(3)) for j in range(6)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    o_bf = [math.fsum(w[j] * v[j, t] for j in range(6)) / l for t in range(3)]
    for causal in (False, True):
        o, lse = attention_rect(q, k, v, causal, 0.5)
        np.testing.assert_allclose(o[0], o_bf, rtol=1e-13, atol=1e-14)
        assert abs(lse[0] - (m + math.log(l))) < 1e-12


def test_rect_default_start_is_end_aligned():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((7, 8)), rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    o, lse = attention_rect(q, k, v, True, 0.4)
    o2, lse2 = attention_rect(q, k, v, True, 0.4, q_start=23)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("q_start", [0, 5, 33, 60])
def test_rect_middle_range_matches_torch_with_explicit_mask(q_start):
    # queries at positions q_start .. q_start + nq - 1 of a 70-key sequence: torch's float64 SDPA with
    # the boolean mask "key j visible to query i iff j <= q_start + i" written out independently
    rng = np.random.default_rng(5 + q_start)
    nq, nk, d = 10, 70, 16
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    mask = torch.zeros((nq, nk), dtype=torch.bool)
    for i in range(nq):
        mask[i, : q_start + i + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                                           attn_mask=mask, scale=0.25)
    o, _ = attention_rect(q, k, v, True, 0.25, q_start=q_start)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rect_middle_range_brute_force():
    # query at position 2 of a 9-key sequence sees exactly keys 0, 1, 2
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((1, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    s = [0.7 * math.fsum(q[0, t] * k[j, t] for t in range(4)) for j in range(3)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    o_bf = [math.fsum(w[j] * v[j, t] for j in range(3)) / l for t in range(4)]
    o, lse = attention_rect(q, k, v, True, 0.7, q_start=2)
    np.testing.assert_allclose(o[0], o_bf, rtol=1e-13, atol=1e-14)
    assert abs(lse[0] - (m + math.log(l))) < 1e-12


def test_rect_shards_reassemble_square_causal():
    # a causal sequence cut into query ranges: each range against all keys, starting at its own
    # position, gives the rows of the square causal attention (the sequence-sharded forward)
    rng = np.random.default_rng(7)
    n, d = 48, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o_sq, lse_sq = attention_rows(q, k, v, np.arange(n), True, 0.35)
    for a, b in [(0, 12), (12, 13), (13, 40), (40, 48)]:
        o, lse = attention_rect(q[a:b], k, v, True, 0.35, q_start=a)
        np.testing.assert_allclose(o, o_sq[a:b], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, lse_sq[a:b], rtol=1e-13, atol=1e-13)


def test_rect_more_queries_than_keys_non_causal():
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((50, 16)), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                                           scale=0.3)
    o, _ = attention_rect(q, k, v, False, 0.3)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)

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

"""Pins of the oracle's materialised score / probability matrices (attention_probs) — CPU only."""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention_probs, attention_rows


@pytest.mark.parametrize("causal", [False, True])
def test_probs_brute_force(causal):
    rng = np.random.default_rng(11)
    n, d, scale = 6, 5, 0.37
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    s, p, lse = attention_probs(q, k, causal, scale)
    for i in range(n):
        vis = [j for j in range(n) if (j <= i or not causal)]
        sij = [scale * math.fsum(q[i, t] * k[j, t] for t in range(d)) for j in range(n)]
        for j in range(n):
            assert abs(s[i, j] - sij[j]) <= 1e-13  # every score, masked or not
        z = math.fsum(math.exp(sij[j]) for j in vis)
        assert abs(lse[i] - math.log(z)) <= 1e-13
        for j in range(n):
            want = math.exp(sij[j]) / z if j in vis else 0.0
            assert abs(p[i, j] - want) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_probs_match_torch_softmax_and_scipy(causal):
    rng = np.random.default_rng(12)
    n, d, scale = 50, 16, 0.25
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    s, p, lse = attention_probs(q, k, causal, scale)
    st = torch.tensor(q) @ torch.tensor(k).T * scale
    if causal:
        st = st.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(p, torch.softmax(st, dim=-1).numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, logsumexp(st.numpy(), axis=1), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_probs_consistent_with_attention_rows(causal):
    rng = np.random.default_rng(13)
    n, d, scale = 40, 8, 0.5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    _, p, lse = attention_probs(q, k, causal, scale)
    o, lse2 = attention_rows(q, k, v, np.arange(n), causal, scale)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0.0)
    np.testing.assert_allclose(p @ v, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)

"""Pins of the backward oracle (the gradients of the attention definition) — CPU only.

The pages give no worked example of the backward pass; the pins are the mathematics: central finite
differences of the forward oracle, torch's float64 autograd through its own scaled_dot_product_attention
(an independent library routine), a closed form (one key) and two invariants of the softmax gradient.
"""

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_ref


def _loss(q, k, v, g, causal, scale):
    o, _ = attention_ref(q, k, v, causal, scale)
    return float((o * g).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_central_differences(causal):
    rng = np.random.default_rng(7 + causal)
    n, d, scale = 5, 4, 0.6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, causal, scale)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            lp = _loss(**{**args, name: xp}, g=g, causal=causal, scale=scale)
            lm = _loss(**{**args, name: xm}, g=g, causal=causal, scale=scale)
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd(causal):
    rng = np.random.default_rng(11)
    b, h, n, d, scale = 2, 3, 37, 16, 0.3
    q, k, v, g = (rng.standard_normal((b, h, n, d)) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(g))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, causal, scale)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_single_key_closed_form():
    # one key and one query: P = 1, so dV = dO and the score gradient vanishes (dQ = dK = 0)
    rng = np.random.default_rng(3)
    q, k, v, g = (rng.standard_normal((1, 8)) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, False, 0.5)
    np.testing.assert_allclose(dv, g, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    # rows of P sum to 1, so sum_j dV_j = sum_i dO_i; rows of dS sum to 0, so sum_j dK_j = 0
    rng = np.random.default_rng(5)
    n, d = 23, 8
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, causal, 0.4)
    np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)

"""Plain float64 scaled-dot-product attention (test infrastructure only).

Definition followed (FlashAttention 2 + 3 — speicherbewusste Attention-Kernels, "Kernpunkte": the
tiled kernel returns exactly what softmax(Q K^T / sqrt(d)) V returns; "Worum es geht": it is not a
different formula, only a different data movement).  For one (batch, head), query row i and the
visible key set J(i) = {0..N-1} (non-causal) or {0..i} (causal, lower-triangular):

    s_ij = scale * sum_t Q[i,t] K[j,t]                  for j in J(i)
    m_i  = max_j s_ij
    l_i  = sum_j exp(s_ij - m_i)
    O_i  = sum_j exp(s_ij - m_i) V[j] / l_i
    lse_i = m_i + ln l_i

Subtracting m_i is the algebraic identity exp(s - m)/sum exp(s - m) = exp(s)/sum exp(s), used only so
that exp never overflows.  Each query row is computed from its full score row in one step: no
splitting of the keys into tiles and no running maximum (that is what the GPU kernel does instead).
All arithmetic is float64 on the exact (already rounded) input values.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or CPU torch tensor (any float dtype) to float64."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def attention_rows(qh, kh, vh, rows, causal: bool, scale: float):
    """Attention output and lse for selected query rows of ONE head.

    qh: [N, d] queries, kh/vh: [N, d] keys/values, rows: 1-D integer array of query indices.
    Returns (O [len(rows), d] float64, lse [len(rows)] float64).
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    rows = np.asarray(rows, dtype=np.int64)
    n_keys = kh.shape[0]
    s = float(scale) * (qh[rows] @ kh.T)  # [r, N]
    if causal:
        visible = np.arange(n_keys)[None, :] <= rows[:, None]
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)  # exp(-inf) = 0 for hidden keys
    l = e.sum(axis=1, keepdims=True)
    o = (e @ vh) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_ref(q, k, v, causal: bool, scale: float, row_chunk: int = 1024):
    """Full attention for tensors [..., N, d] (leading dims = batch, heads).

    Returns (O float64 [..., N, d], lse float64 [..., N]).  Query rows are processed in chunks of
    ``row_chunk`` only to bound memory; every chunk sees all of its keys at once.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, d = q.shape[-2], q.shape[-1]
    o = np.empty(lead + (n, v.shape[-1]), dtype=np.float64)
    lse = np.empty(lead + (n,), dtype=np.float64)
    for idx in np.ndindex(*lead):
        for r0 in range(0, n, row_chunk):
            rows = np.arange(r0, min(n, r0 + row_chunk))
            o_c, lse_c = attention_rows(q[idx], k[idx], v[idx], rows, causal, scale)
            o[idx][r0:r0 + len(rows)] = o_c
            lse[idx][r0:r0 + len(rows)] = lse_c
    return o, lse


def attention_bwd_rows(qh, kh, vh, doh, causal: bool, scale: float):
    """Gradients of the attention definition for ONE head: returns (dQ, dK, dV) float64 [N, d].

    The pages name the backward pass (FlashAttention 2 + 3 — speicherbewusste Attention-Kernels,
    "Kernpunkte": FlashAttention 2 parallelises it better) but do not write it out; this is the
    derivative of the definition above, for a loss L whose gradient with respect to O is dO:

        P_ij  = exp(s_ij - lse_i) on visible keys, 0 elsewhere      (the softmax of each row)
        dV    = P^T dO
        dP    = dO V^T
        D_i   = sum_t dO[i,t] O[i,t]          (= sum_j P_ij dP_ij, the row term of the softmax)
        dS_ij = P_ij (dP_ij - D_i)             (softmax derivative, row by row)
        dQ    = scale dS K,   dK = scale dS^T Q

    Full score rows, float64, no tiling.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    n = qh.shape[0]
    s = float(scale) * (qh @ kh.T)
    if causal:
        s = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ vh
    dv = p.T @ doh
    dp = doh @ vh.T
    dd = (doh * o).sum(axis=1, keepdims=True)
    ds = p * (dp - dd)
    dq = float(scale) * (ds @ kh)
    dk = float(scale) * (ds.T @ qh)
    return dq, dk, dv


def attention_bwd_ref(q, k, v, do, causal: bool, scale: float):
    """attention_bwd_rows over leading (batch, head) dims; tensors [..., N, d]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq, dk, dv = (np.empty_like(q), np.empty_like(k), np.empty_like(v))
    for idx in np.ndindex(*q.shape[:-2]):
        dq[idx], dk[idx], dv[idx] = attention_bwd_rows(q[idx], k[idx], v[idx], do[idx], causal, scale)
    return dq, dk, dv


def attention_rect(qh, kh, vh, causal: bool, scale: float, q_start=None):
    """Attention of Nq queries against Nk keys for ONE head, same definition as attention_rows with full
    score rows.  The queries are the positions q_start .. q_start + Nq - 1 of the key sequence: causal
    means query i sees keys j <= q_start + i.  q_start defaults to Nk - Nq (the queries are the last Nq
    positions, the decode shape, mask aligned to the end of the key sequence); with Nq == Nk and
    q_start = 0 this is the lower-triangular mask of attention_rows.  Rows of a query range taken from
    the middle of a sequence (q_start + Nq < Nk) see a prefix of the keys only.  q_start is ignored
    when causal is false.  Returns (O [Nq, d], lse [Nq]) in float64.
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    nq, nk = qh.shape[0], kh.shape[0]
    s = float(scale) * (qh @ kh.T)
    if causal:
        start = nk - nq if q_start is None else int(q_start)
        assert start >= 0, "causal queries start at a key position >= 0"
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + start, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vh) / l, m[:, 0] + np.log(l[:, 0])


def attention_probs(qh, kh, causal: bool, scale: float):
    """The intermediate matrices of the definition for ONE head, as the standard (unfused) implementation
    materialises them: scores s = scale Q K^T [N, N] (all entries, mask not applied), probabilities
    P_ij = exp(s_ij - m_i) / l_i on the visible keys and 0 elsewhere, and lse [N].  float64, full rows
    (concept card "Worum es geht": the classic path holds the whole score matrix)."""
    qh, kh = _f64(qh), _f64(kh)
    n = qh.shape[0]
    s = float(scale) * (qh @ kh.T)
    sm = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], s, -np.inf) if causal else s
    m = sm.max(axis=1, keepdims=True)
    e = np.exp(sm - m)
    l = e.sum(axis=1, keepdims=True)
    return s, e / l, m[:, 0] + np.log(l[:, 0])

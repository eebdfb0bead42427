"""Plain fp64 definition of attention.  TEST INFRASTRUCTURE ONLY (see package
docstring for who may import it).

What is computed ([trading post], "Why attention is bound to memory"; [FA4
post], "Introduction"):  O = softmax(Q K^T * scale) V  per (batch, head),
with scale = 1/sqrt(d_k) by default.  The causal variant fills future
scores with -inf before the softmax ([trading post], "Integration in eight
lines" and "Causal masking").  Besides O the forward pass keeps the softmax
statistics (m, l) of each query row ([trading post], "Backward: recompute
instead of store"); this oracle reports them folded into the natural-log
log-sum-exp LSE = m + ln(l) = ln(sum_j exp(s_ij)) over the visible keys.

Readings where the sources are silent:
  * causal alignment for Nq != Nk is bottom-right: query i sees key j iff
    j <= i + (Nk - Nq), so the newest query sees the whole key range;
    causal with Nq > Nk is rejected (some rows would see no key);
  * rows are independent, so the evaluation walks over row chunks purely to
    bound memory; each row's whole softmax is formed at once.

Parity status: pinned (brute force in 40-digit mpmath, torch's CPU float64
scaled_dot_product_attention, closed forms for uniform and one-hot scores,
permutation/shift invariances, causal prefix identity; tests/test_oracle_*).
"""
from __future__ import annotations

import numpy as np


def softmax_rows(s: np.ndarray):
    """Row softmax of a score matrix: returns (P, m, l) with m the row max,
    l = sum_j exp(s_ij - m), P = exp(s - m) / l."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def attention_head(q, k, v, scale: float, causal: bool = False, row_chunk: int = 1024):
    """One head: q [Nq, d], k [Nk, d], v [Nk, dv] (any real dtype, widened to
    fp64).  Returns (O [Nq, dv] fp64, LSE [Nq] fp64)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    o = np.empty((Nq, v.shape[1]), np.float64)
    lse = np.empty(Nq, np.float64)
    for r0 in range(0, Nq, row_chunk):
        r1 = min(Nq, r0 + row_chunk)
        s = q[r0:r1] @ k.T * float(scale)
        if causal:
            i = np.arange(r0, r1)[:, None]
            j = np.arange(Nk)[None, :]
            s = np.where(j <= i + (Nk - Nq), s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        o[r0:r1] = (e @ v) / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False, row_chunk: int = 1024):
    """Batched [..., N, d] attention; leading dims are independent heads.
    Returns (O fp64 [..., Nq, dv], LSE fp64 [..., Nq])."""
    q = np.asarray(q)
    lead = q.shape[:-2]
    qf = q.reshape((-1,) + q.shape[-2:])
    kf = np.asarray(k).reshape((-1,) + np.asarray(k).shape[-2:])
    vf = np.asarray(v).reshape((-1,) + np.asarray(v).shape[-2:])
    outs, lses = [], []
    for i in range(qf.shape[0]):
        o, l = attention_head(qf[i], kf[i], vf[i], scale, causal, row_chunk)
        outs.append(o)
        lses.append(l)
    o = np.stack(outs).reshape(lead + outs[0].shape)
    lse = np.stack(lses).reshape(lead + lses[0].shape)
    return o, lse


def attention_rows(q, k, v, rows, scale: float, causal: bool = False):
    """Selected query rows of one head (for sampled checks at full size):
    same definition as ``attention_head``, evaluated only for ``rows``.
    The causal mask uses each row's own index in the full Nq range."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    s = q[rows] @ k.T * float(scale)
    if causal:
        j = np.arange(Nk)[None, :]
        s = np.where(j <= rows[:, None] + (Nk - Nq), s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return (e @ v) / l[:, None], m + np.log(l)

"""Plain fp64 gradient of attention.  TEST INFRASTRUCTURE ONLY (see package
docstring for who may import it).

What is computed: given the upstream gradient dO of the forward output
O = softmax(S) V with S = scale * Q K^T (future keys masked to -inf when
causal), the gradients dQ, dK, dV of the scalar sum(dO * O).  The [trading
post] ("Backward: recompute instead of store") says the backward pass
rebuilds the probability tiles from Q and K instead of storing them, keeping
only O and the softmax statistics; it does not print the gradient formulas,
so this module writes out the chain rule through the definition:

    P  = softmax(S)                       (row-wise, masked entries 0)
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))        (Jacobian of the row softmax)
    dQ = scale * dS K
    dK = scale * dS^T Q

The softmax Jacobian term is evaluated as rowsum(P * dP) here, straight from
the definition; a kernel may use the equal quantity rowsum(dO * O).  Rows are
independent, so they are walked in chunks only to bound memory.

Parity status: pinned (central finite differences of sum(dO * O) through the
forward definition, torch's CPU float64 autograd of the plain expression,
closed forms for uniform scores, the zero-sum and key-shift invariants;
tests/test_oracle_backward.py).
"""
from __future__ import annotations

import numpy as np


def attention_backward_head(q, k, v, do, scale: float, causal: bool = False, row_chunk: int = 512):
    """One head: q [Nq, d], k [Nk, d], v [Nk, dv], do [Nq, dv] (any real dtype,
    widened to fp64).  Returns (dQ [Nq, d], dK [Nk, d], dV [Nk, dv]) in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, Nq, row_chunk):
        r1 = min(Nq, r0 + row_chunk)
        s = q[r0:r1] @ k.T * float(scale)
        if causal:
            i = np.arange(r0, r1)[:, None]
            j = np.arange(Nk)[None, :]
            s = np.where(j <= i + (Nk - Nq), s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        p = e / e.sum(axis=1)[:, None]
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        dq[r0:r1] = float(scale) * (ds @ k)
        dk += float(scale) * (ds.T @ q[r0:r1])
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float, causal: bool = False, row_chunk: int = 512):
    """Batched [..., N, d]; leading dims are independent heads.  Returns
    (dQ, dK, dV) in fp64 with the shapes of q, k, v."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    qf = q.reshape((-1,) + q.shape[-2:])
    kf = k.reshape((-1,) + k.shape[-2:])
    vf = v.reshape((-1,) + v.shape[-2:])
    dof = do.reshape((-1,) + do.shape[-2:])
    dqs, dks, dvs = [], [], []
    for i in range(qf.shape[0]):
        a, b, c = attention_backward_head(qf[i], kf[i], vf[i], dof[i], scale, causal, row_chunk)
        dqs.append(a)
        dks.append(b)
        dvs.append(c)
    return (np.stack(dqs).reshape(q.shape), np.stack(dks).reshape(k.shape), np.stack(dvs).reshape(v.shape))

"""Grouped-query heads and packed variable-length batches, in fp64.  TEST
INFRASTRUCTURE ONLY (see package docstring for who may import it).

The [FA4 post] lists grouped-query attention (GQA, and MQA as its one-group
case) and variable-length ("varlen") batches among the features missing from
FA4's forward; it defines neither.  Readings (the plainest ones):

  * GQA: H query heads share Hkv = H / g key/value heads; query head h
    attends with K/V head h // g (consecutive query heads share a K/V head).
    MQA is Hkv = 1.  Each query head's attention is otherwise the plain
    definition (oracle.attention).
  * varlen: several sequences of different lengths packed along the token
    axis, located by cumulative offsets cu_q = [0, n_0, n_0 + n_1, ...] (and
    cu_k for the keys).  Tensors are head-major, [H, total, d] (one head's
    tokens of every sequence back to back), LSE is [H, total_q].  Sequence s
    is plain attention of its own queries over its own keys; the causal mask
    is bottom-right aligned within each sequence.  A query that sees no key
    (an empty key range, or causal with more queries than keys) has O = 0 and
    LSE = -inf by this reading: the sum over an empty set of keys.

Every function reduces to the pinned dense oracle by slicing and head
mapping only; no arithmetic of its own.

Gradients (the backward pass, [trading post] "Backward: recompute instead of
store"): dQ per query head; dK, dV of a shared K/V head are the sums over the
query heads that read it; in a packed batch each sequence is its own
problem, and a query row that sees no key has O = 0 whatever its inputs, so
it contributes no gradient.

Parity status: pinned (GQA equals dense attention with K/V heads repeated
explicitly and torch's CPU float64 scaled_dot_product_attention with
enable_gqa; varlen equals one dense call per sequence; empty rows; GQA
gradients against torch autograd through repeat_interleave; varlen
gradients against one dense backward per sequence and finite differences;
tests/test_oracle_variants.py).
"""
from __future__ import annotations

import numpy as np

from . import attention as A
from . import backward as BW


def kv_head(h: int, H: int, Hkv: int) -> int:
    """The K/V head that query head h reads (consecutive groups of H/Hkv)."""
    if Hkv < 1 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    return h // (H // Hkv)


def attention_gqa(q, k, v, scale: float, causal: bool = False):
    """q [B, H, Nq, d], k, v [B, Hkv, Nk, d] -> (O [B, H, Nq, dv], LSE [B, H, Nq]) fp64."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    O = np.empty(q.shape[:3] + (v.shape[3],))
    L = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            O[b, h], L[b, h] = A.attention_head(q[b, h], k[b, g], v[b, g], scale, causal)
    return O, L


def _seq_attention(q, k, v, scale, causal):
    """One sequence of one head; rows that see no key give O = 0, LSE = -inf."""
    Nq, Nk = q.shape[0], k.shape[0]
    O = np.zeros((Nq, v.shape[1]))
    L = np.full(Nq, -np.inf)
    if Nq == 0 or Nk == 0:
        return O, L
    if causal and Nq > Nk:
        # rows i < Nq - Nk see no key; the rest are causal attention over all keys
        first = Nq - Nk
        O[first:], L[first:] = A.attention_head(q[first:], k, v, scale, True)
        return O, L
    return A.attention_head(q, k, v, scale, causal)


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False):
    """q [H, total_q, d], k, v [Hkv, total_k, d] with sequence offsets cu_q,
    cu_k (length nseq + 1) -> (O [H, total_q, dv], LSE [H, total_q]) fp64."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    H, Hkv = q.shape[0], k.shape[0]
    O = np.zeros(q.shape[:2] + (v.shape[2],))
    L = np.full(q.shape[:2], -np.inf)
    for s in range(len(cu_q) - 1):
        qa, qb = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        for h in range(H):
            g = kv_head(h, H, Hkv)
            O[h, qa:qb], L[h, qa:qb] = _seq_attention(q[h, qa:qb], k[g, ka:kb], v[g, ka:kb], scale, causal)
    return O, L


def attention_backward_gqa(q, k, v, do, scale: float, causal: bool = False):
    """Gradients for GQA: dQ per query head; dK, dV of a K/V head are the sums
    over the query heads that read it (the chain rule through the shared
    head).  Shapes as in attention_gqa."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    dq = np.empty(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            a, bk, bv = BW.attention_backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dq[b, h] = a
            dk[b, g] += bk
            dv[b, g] += bv
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, scale: float, causal: bool = False):
    """Gradients of sum(dO * O) for attention_varlen: q, do [H, total_q, d],
    k, v [Hkv, total_k, d]; returns (dQ, dK, dV) fp64 with those shapes."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    H, Hkv = q.shape[0], k.shape[0]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for s in range(len(cu_q) - 1):
        qa, qb = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        Nq, Nk = qb - qa, kb - ka
        if Nq == 0 or Nk == 0:
            continue
        # rows that see no key (causal, Nq > Nk) have a constant O = 0
        first = Nq - Nk if (causal and Nq > Nk) else 0
        for h in range(H):
            g = kv_head(h, H, Hkv)
            a, bk, bv = BW.attention_backward_head(q[h, qa + first:qb], k[g, ka:kb], v[g, ka:kb],
                                                   do[h, qa + first:qb], scale, causal)
            dq[h, qa + first:qb] = a
            dk[g, ka:kb] += bk
            dv[g, ka:kb] += bv
    return dq, dk, dv

"""The tiled online-softmax recurrence, in fp64.  TEST INFRASTRUCTURE ONLY.

``flash_forward_tiled`` takes the steps of [trading post], "The Flash
Attention algorithm", in that section's order and notation: Q is cut into
T_r = ceil(N/B_r) row blocks Q_i and K, V into T_c = ceil(N/B_c) column
blocks K_j, V_j.  For each query block the state O_i = 0, m_i = -inf,
l_i = 0 is carried across the key blocks:

    S_ij  = Q_i K_j^T * scale
    m_ij  = rowmax(S_ij)
    P_ij  = exp(S_ij - m_ij)
    l_ij  = rowsum(P_ij)
    m_new = max(m_i, m_ij)
    l_new = exp(m_i - m_new) l_i + exp(m_ij - m_new) l_ij
    O_i   = (l_i exp(m_i - m_new) / l_new) O_i + (exp(m_ij - m_new) / l_new) P_ij V_j
    m_i, l_i = m_new, l_new

i.e. the output is renormalised after every block (the form of the first
FlashAttention).  "The online softmax recurrence" states that the result is
algebraically the two-pass softmax; the tests hold this function to the plain
definition in ``oracle.attention`` at 1e-12.

Readings where the section is silent:
  * a tile row whose keys are all masked has m_ij = -inf; it contributes
    nothing (P_ij = 0, l_ij = 0) instead of exp(-inf - -inf) = NaN;
  * LSE is m + ln(l) of the final state (the stored (m, l) statistics of
    "Backward: recompute instead of store").

``merge_states`` combines partial results computed over disjoint key ranges.
It is the same update as the last two lines above, applied to states that
are already normalised: with L_s = m_s + ln l_s, the merged state is
L = M + ln sum_s exp(L_s - M) (M = max_s L_s) and O = sum_s exp(L_s - L) O_s.
A state whose range saw no visible key has L_s = -inf and weight 0.

Parity status: pinned (equality with the two-pass definition for several
block sizes and masks; split-and-merge equality with the whole-range result).
"""
from __future__ import annotations

import math

import numpy as np


def flash_forward_tiled(q, k, v, scale: float, causal: bool = False,
                        B_r: int = 16, B_c: int = 16):
    """One head, q [Nq, d], k [Nk, d], v [Nk, dv].  Returns (O, LSE) fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    T_r = math.ceil(Nq / B_r)
    T_c = math.ceil(Nk / B_c)
    O = np.zeros((Nq, v.shape[1]))
    LSE = np.zeros(Nq)
    for i in range(T_r):
        rows = np.arange(i * B_r, min(Nq, (i + 1) * B_r))
        Q_i = q[rows]
        O_i = np.zeros((len(rows), v.shape[1]))
        m_i = np.full(len(rows), -np.inf)
        l_i = np.zeros(len(rows))
        for j in range(T_c):
            cols = np.arange(j * B_c, min(Nk, (j + 1) * B_c))
            K_j, V_j = k[cols], v[cols]
            S_ij = Q_i @ K_j.T * float(scale)
            if causal:
                S_ij = np.where(cols[None, :] <= rows[:, None] + (Nk - Nq), S_ij, -np.inf)
            m_ij = S_ij.max(axis=1)
            live = np.isfinite(m_ij)
            m_ref = np.where(live, m_ij, 0.0)
            P_ij = np.where(live[:, None], np.exp(S_ij - m_ref[:, None]), 0.0)
            l_ij = P_ij.sum(axis=1)
            m_new = np.maximum(m_i, m_ij)
            # exp(-inf - finite) = 0; rows still without any visible key keep l = 0
            a_old = np.where(np.isfinite(m_i), np.exp(m_i - np.where(np.isfinite(m_new), m_new, 0.0)), 0.0)
            a_new = np.where(live, np.exp(m_ij - np.where(np.isfinite(m_new), m_new, 0.0)), 0.0)
            l_new = l_i * a_old + l_ij * a_new
            safe = np.where(l_new > 0, l_new, 1.0)
            O_i = O_i * (l_i * a_old / safe)[:, None] + (P_ij @ V_j) * (a_new / safe)[:, None]
            m_i, l_i = m_new, l_new
        O[rows] = O_i
        LSE[rows] = m_i + np.log(l_i)
    return O, LSE


def merge_states(O_parts, LSE_parts):
    """Merge normalised partial states (O_s [S, ..., dv], LSE_s [S, ...]) over
    disjoint key ranges into (O, LSE)."""
    O_parts = np.asarray(O_parts, np.float64)
    L = np.asarray(LSE_parts, np.float64)
    M = L.max(axis=0)
    Mref = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(L - Mref)                      # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    lse = Mref + np.log(tot)
    wn = np.where(np.isfinite(L), np.exp(L - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
    O = (wn[..., None] * O_parts).sum(axis=0)
    return O, lse


def split_kv_forward(q, k, v, scale: float, bounds, partial_fn):
    """Attention of one head by key ranges [bounds[s], bounds[s+1]), each
    evaluated by ``partial_fn(q, k_s, v_s, scale)`` -> (O_s, LSE_s), then
    merged with ``merge_states``.  Non-causal only (each range must be
    non-empty)."""
    Os, Ls = [], []
    for s in range(len(bounds) - 1):
        a, b = bounds[s], bounds[s + 1]
        o, l = partial_fn(q, k[a:b], v[a:b], scale)
        Os.append(o)
        Ls.append(l)
    return merge_states(np.stack(Os), np.stack(Ls))

"""The online-softmax recurrence, in fp64.  TEST INFRASTRUCTURE ONLY (see the
package docstring for who may import it).

``online_forward`` evaluates attention the way a tiled kernel has to: it never
holds a whole score row, only one block of keys at a time, and carries three
running quantities per query row across the key blocks:

  * ``top``  -- the largest visible score seen so far (-inf before any);
  * ``mass`` -- the sum of exp(score - top) over the keys seen so far;
  * ``acc``  -- the sum of exp(score - top) * v over the same keys.

When a new block raises ``top``, the history is brought to the new reference
by one factor exp(top_old - top_new); that is the rescaling of "The online
softmax recurrence" in [trading post] (an accumulated output is scaled down
as if the new maximum had been known from the start).  The division by the
total mass is left to the very end, the deferred normalisation that the
"FA2" section of the same post gives as its first change (fewer non-matmul
operations in the inner loop).  Splitting Q into row blocks and K, V into key
blocks follows "The Flash Attention algorithm"; the block sizes are free
parameters, and "The online softmax recurrence" says the result is the
two-pass softmax in exact arithmetic, which the tests hold this function to
(``oracle.attention`` at 1e-12 for many block shapes).

Readings where the pages are silent:
  * a row that has not yet seen a visible key keeps top = -inf and zero mass
    and accumulator; exp(-inf) = 0 is used for both its history factor and
    its masked scores, so no NaN arises from -inf - -inf;
  * LSE is top + ln(mass) of the final state: the stored softmax statistics
    (m, l) of "Backward: recompute instead of store", folded into one number.

``merge_states`` combines normalised partial results computed over disjoint
key ranges (the split-KV decode): with L_s = ln of each part's mass plus its
top, the merged L = M + ln sum_s exp(L_s - M) (M = max_s L_s) and
O = sum_s exp(L_s - L) O_s, the same rescale-and-add step applied to whole
ranges; a part that saw no visible key has L_s = -inf and weight 0.

Parity status: pinned (equality with the two-pass definition for several
block shapes and masks, the definition's own closed-form pins, planted
mistakes in tests/test_oracle_mutations.py; split-and-merge equality with the
whole-range result).
"""
from __future__ import annotations

import numpy as np


def online_forward(q, k, v, scale: float, causal: bool = False,
                   rows_per_block: int = 16, keys_per_block: int = 16):
    """One head, q [Nq, d], k [Nk, d], v [Nk, dv].  Returns (O, LSE) fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    out = np.empty((Nq, v.shape[1]))
    lse = np.empty(Nq)
    for r0 in range(0, Nq, rows_per_block):
        qrows = np.arange(r0, min(Nq, r0 + rows_per_block))
        top = np.full(len(qrows), -np.inf)
        mass = np.zeros(len(qrows))
        acc = np.zeros((len(qrows), v.shape[1]))
        for c0 in range(0, Nk, keys_per_block):
            keys = np.arange(c0, min(Nk, c0 + keys_per_block))
            block = (q[qrows] @ k[keys].T) * float(scale)
            if causal:
                future = keys[None, :] > qrows[:, None] + (Nk - Nq)
                block = np.where(future, -np.inf, block)
            new_top = np.maximum(top, block.max(axis=1))
            ref = np.where(np.isfinite(new_top), new_top, 0.0)
            history = np.exp(top - ref)
            weights = np.exp(block - ref[:, None])
            mass = mass * history + weights.sum(axis=1)
            acc = acc * history[:, None] + weights @ v[keys]
            top = new_top
        out[qrows] = acc / mass[:, None]
        lse[qrows] = top + np.log(mass)
    return out, lse


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

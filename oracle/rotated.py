"""Rotated FP8 attention (incoherent processing), in emulation.  TEST
INFRASTRUCTURE ONLY (see package docstring for who may import it).

The [trading post], section "FA3: Hopper mechanisms", item "FP8 with
incoherent processing": naive FP8 attention is ruined by outliers, so FA3
multiplies the vectors by a random rotation before block quantisation, which
spreads an outlier's magnitude over all coordinates; the page reports 2.6x
lower numerical error than naive FP8.  The page fixes neither the rotation,
the block size nor what happens to V and P.  Readings (the plainest ones):

  * the rotation is R = diag(sigma) H_d / sqrt(d): H_d the Sylvester Hadamard
    matrix (H_1 = [1], H_2n = [[H, H], [H, -H]]), sigma a vector of random
    signs drawn once and passed in; R is orthogonal, so (Q R)(K R)^T = Q K^T
    and only Q and K are rotated (V is not: rotating it would change O);
  * x R is evaluated in fp32 as the fast Walsh-Hadamard transform of
    x * sigma, butterflies (lo, hi) -> (lo + hi, lo - hi) at strides
    1, 2, 4, ..., d/2 in that order, with the 1/sqrt(d) folded into the
    stored scale (the quantisation codes are decided on the unnormalised
    transform y' = (x * sigma) H_d, in fp32);
  * block quantisation: consecutive rows of one head form blocks of
    ``block_rows`` rows (the last block of a head may be shorter); a block's
    scale is s' = max|y'| / 448 in fp32, its codes E4M3(y' / s') (fp32
    division, OCP E4M3FN, ties to even, saturating); the stored per-row scale
    is fp32(s' * fp32(1 / sqrt(d))); a zero block gets scale 0 and codes 0.
    Without rotation (sigma = None) y' = x and the stored scale is s';
  * V: per-tensor E4M3 and P: E4M3, as in the quantised forward of
    oracle.quant (steps 2, 5, 6 there); the scores are the exact products of
    the decoded codes times the two row scales times the softmax scale.

Parity status: pinned.  The Hadamard matrix against scipy.linalg.hadamard
and H H^T = d I; the fp32 transform against the integer product x H_d on
integer inputs (exact in fp32) and its own inverse; rotation invariance of
Q K^T; block quantisation without rotation against oracle.quant's pinned
per-tensor E4M3 applied block by block; the one-hot closed form; the
attention against oracle.quant's pinned int8 form on integer codes, the
uniform-score closed form, and the method's own claim (lower error than
unrotated FP8 on inputs with outliers) (tests/test_oracle_rotated.py).
"""
from __future__ import annotations

import numpy as np

from . import quant as Q


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (d a power of two), int64 entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1), np.int64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def fwht_f32(x) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the rows of x ([..., d]) in
    fp32: x H_d, evaluated by butterflies at strides 1, 2, ..., d/2."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        lo = z[..., 0, :].copy()
        hi = z[..., 1, :].copy()
        z[..., 0, :] = lo + hi        # fp32 adds, each correctly rounded
        z[..., 1, :] = lo - hi
        y = z.reshape(lead + (d,))
        h *= 2
    return y


def rotate_quantize_e4m3(x32, signs, block_rows: int):
    """x32 [..., N, d] fp32 (the bf16 inputs widened) -> (codes uint8
    [..., N, d], per-row scales fp32 [..., N]) by the readings above;
    ``signs`` is a length-d array of +-1, or None for no rotation."""
    x32 = np.asarray(x32, dtype=np.float32)
    if block_rows < 1:
        raise ValueError("block_rows must be positive")
    N, d = x32.shape[-2:]
    if signs is None:
        y, post = x32, None
    else:
        s = np.asarray(signs, np.float32)
        if s.shape != (d,) or not np.all(np.abs(s) == 1):
            raise ValueError("signs must be d values of +-1")
        y, post = fwht_f32(x32 * s), np.float32(1.0 / np.sqrt(d))
    codes = np.zeros(y.shape, np.uint8)
    scales = np.zeros(y.shape[:-1], np.float32)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        blk = y[..., r0:r1, :]
        amax = np.max(np.abs(blk), axis=(-2, -1)).astype(np.float32)
        sc = (amax / np.float32(Q.E4M3_MAX)).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1)).astype(np.float32)
        c = Q.e4m3_encode((blk / safe[..., None, None]).astype(np.float32))
        codes[..., r0:r1, :] = np.where((sc > 0)[..., None, None], c, 0)
        row_scale = sc if post is None else (sc * post).astype(np.float32)
        scales[..., r0:r1] = row_scale[..., None]
    return codes, scales


def attention_fp8_head(q8, sq, k8, sk, v8, sv, scale: float, causal: bool = False):
    """FP8 attention of one head from E4M3 codes: S = decode(q8) decode(k8)^T
    * sq[i] * sk[j] * scale (exact products, fp64), mask, P = exp(S - m),
    l = sum P, O = (E4M3(P) . decode(v8) * sv) / l.  Returns (O, LSE) fp64."""
    Nq, Nk = q8.shape[0], k8.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    s = Q.e4m3_decode(q8) @ Q.e4m3_decode(k8).T
    s = s * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * float(scale)
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        s = np.where(j <= i + (Nk - Nq), s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    p_q = Q.e4m3_decode(Q.e4m3_encode(p))
    return (p_q @ (Q.e4m3_decode(v8) * float(sv))) / l[:, None], m + np.log(l)


def quantize_inputs(q32, k32, v32, signs, block_rows: int):
    """Q and K rotated (if signs is not None) and block-quantised, V per
    tensor: dict(q8, sq, k8, sk, v8, sv)."""
    q8, sq = rotate_quantize_e4m3(q32, signs, block_rows)
    k8, sk = rotate_quantize_e4m3(k32, signs, block_rows)
    v8, sv = Q.quantize_per_tensor_e4m3(v32)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv)


def attention_rotated_fp8(q32, k32, v32, signs, scale: float, causal: bool = False, block_rows: int = 64):
    """The whole rotated FP8 forward on [..., N, d] tensors.  Returns
    (O, LSE, quantised inputs)."""
    qi = quantize_inputs(q32, k32, v32, signs, block_rows)
    lead = np.asarray(q32).shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    shp = lambda a: a.reshape((n,) + a.shape[len(lead):])
    q8, sq, k8, sk, v8 = (shp(qi[x]) for x in ("q8", "sq", "k8", "sk", "v8"))
    outs, lses = [], []
    for i in range(n):
        o, l = attention_fp8_head(q8[i], sq[i], k8[i], sk[i], v8[i], qi["sv"], scale, causal)
        outs.append(o)
        lses.append(l)
    O = np.stack(outs).reshape(lead + outs[0].shape)
    L = np.stack(lses).reshape(lead + lses[0].shape)
    return O, L, qi

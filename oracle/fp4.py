"""FP8 attention with the probabilities P in MXFP4, in emulation.  TEST
INFRASTRUCTURE ONLY (see package docstring for who may import it).

The [FP4 summary] ("Hardware-Aware FP4 FlashAttention-4", summary and
explainer) runs attention's matrix products in four-bit floating point and
names the conversion of scores to four-bit probabilities as the bottleneck
it removes ("Direct-P": the scores are mapped straight to the hardware's
four-bit encoding of P instead of computing P and then scaling and rounding
it).  It gives no formulas.  Readings (the plainest ones):

  * the four-bit format is OCP E2M1 (1 sign, 2 exponent bits with bias 1,
    1 mantissa bit): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; encoding rounds
    to nearest with ties to the even code and saturates at 6;
  * the hardware's block scaling is OCP MX: for each query row, every block
    of 32 consecutive keys (starting at key 0) shares one power-of-two scale
    2^e with e = floor(log2(max P of the block)) - 2, which puts the block's
    largest P in E2M1's top binade [4, 8); P~ = E2M1(P / 2^e) * 2^e; a block
    whose P are all 0 stays 0;
  * "mapping scores straight to the encoding" yields the same code as
    rounding the exact P = exp(S - m) (the code is a monotone step function
    of S - m with steps at the logarithms of the midpoints), so the oracle
    rounds the exact P;
  * P is the tiled recurrence's own P ([trading post], "The Flash Attention
    algorithm" and "The online softmax recurrence"): keys are taken in
    tiles of ``tile`` keys; for each tile the running max m is raised to
    include it, the accumulated O and l are rescaled by exp(m_old - m_new),
    and the tile's P = exp(S - m) is quantised before its product with V.
    With a four-bit P the max it is taken against matters (a block's scale
    and the rounding points move with it), so the tile width is a parameter
    (the GPU kernel's is 64 keys); MX blocks are 32 consecutive keys from the
    tile's start;
  * l sums the unquantised P, as in the quantised forward; Q, K are E4M3
    with per-row scales and V per-tensor E4M3, as in oracle.rotated (the
    scores are exact products of the decoded codes).

Parity status: pinned.  The E2M1 table against the format's closed form,
encoding at every value, midpoint and neighbour; the block quantisation
against closed forms (powers of two, the 1/16 cut-off, saturation-free
block maxima) and against a per-element brute force over the eight codes;
the attention against the uniform and one-dominant-key closed forms and
against oracle.rotated's FP8 attention where every P is exact in both
formats; the recurrence, with the quantiser replaced by the identity,
against the plain definition for several tile widths
(tests/test_oracle_fp4.py).
"""
from __future__ import annotations

import numpy as np

from . import quant as Q
from . import rotated as RT

E2M1_MAX = 6.0
MX_BLOCK = 32

# non-negative magnitudes in code order 0 .. 7 (monotonic)
_E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 code (0 .. 15, bit 3 the sign) -> value (fp64)."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(c & 8, -1.0, 1.0) * mag


def e2m1_encode(x) -> np.ndarray:
    """Value -> E2M1 code: round to nearest, ties to the even code,
    saturating at 6; ``x`` is taken exactly."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    t = _E2M1_TABLE
    hi = np.clip(np.searchsorted(t, a, side="left"), 1, len(t) - 1)
    lo = hi - 1
    mid = (t[lo] + t[hi]) * 0.5
    code = np.where(a < mid, lo, np.where(a > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == 0.0, 0, code)
    code = np.where(a >= E2M1_MAX, 7, code)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def quantize_p_mx(p, block: int = MX_BLOCK) -> np.ndarray:
    """P [Nq, Nk] >= 0 -> the dequantised MXFP4 P~ (fp64): per row, blocks of
    ``block`` consecutive keys share 2^e, e = floor(log2 max) - 2."""
    p = np.asarray(p, dtype=np.float64)
    Nq, Nk = p.shape
    nb = -(-Nk // block)
    pp = np.zeros((Nq, nb * block))
    pp[:, :Nk] = p
    pb = pp.reshape(Nq, nb, block)
    pmax = pb.max(axis=2)
    # floor(log2 pmax) exactly: pmax = f 2^E with f in [0.5, 1)
    _, E = np.frexp(np.where(pmax > 0, pmax, 1.0))
    e = (E - 1 - 2).astype(np.float64)
    y = pb / np.exp2(e)[:, :, None]                  # exact: a power of two
    out = e2m1_decode(e2m1_encode(y)) * np.exp2(e)[:, :, None]
    out = np.where((pmax > 0)[:, :, None], out, 0.0)
    return out.reshape(Nq, nb * block)[:, :Nk]


def attention_fp4p_head(q8, sq, k8, sk, v8, sv, scale: float, causal: bool = False, tile: int = 64,
                        quantize=quantize_p_mx):
    """One head: scores from E4M3 codes (exact products) * sq[i] * sk[j] *
    scale, masked; then the tiled recurrence, each tile's P quantised by
    ``quantize`` (MXFP4) before its product with decode(v8) * sv; l sums the
    unquantised P.  Returns (O, LSE) fp64."""
    Nq, Nk = q8.shape[0], k8.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    if tile < 1:
        raise ValueError("tile must be positive")
    s = Q.e4m3_decode(q8) @ Q.e4m3_decode(k8).T
    s = s * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * float(scale)
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        s = np.where(j <= i + (Nk - Nq), s, -np.inf)
    vd = Q.e4m3_decode(v8) * float(sv)
    m = np.full(Nq, -np.inf)
    l = np.zeros(Nq)
    acc = np.zeros((Nq, vd.shape[1]))
    for t0 in range(0, Nk, tile):
        st = s[:, t0:t0 + tile]
        m_new = np.maximum(m, st.max(axis=1))
        alpha = np.where(m == -np.inf, 0.0, np.exp(m - np.where(m_new == -np.inf, 0.0, m_new)))
        p = np.where(st == -np.inf, 0.0, np.exp(st - np.where(m_new == -np.inf, 0.0, m_new)[:, None]))
        l = l * alpha + p.sum(axis=1)
        acc = acc * alpha[:, None] + quantize(p) @ vd[t0:t0 + tile]
        m = m_new
    return acc / l[:, None], m + np.log(l)


def attention_fp4p(q32, k32, v32, signs, scale: float, causal: bool = False, block_rows: int = 64,
                   tile: int = 64):
    """The whole forward on [..., N, d] tensors: Q and K rotated (signs, or
    None) and block-quantised to E4M3 as oracle.rotated, V per-tensor E4M3,
    P in MXFP4.  Returns (O, LSE, quantised inputs)."""
    qi = RT.quantize_inputs(q32, k32, v32, signs, block_rows)
    lead = np.asarray(q32).shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    shp = lambda a: a.reshape((n,) + a.shape[len(lead):])
    q8, sq, k8, sk, v8 = (shp(qi[x]) for x in ("q8", "sq", "k8", "sk", "v8"))
    outs, lses = [], []
    for i in range(n):
        o, l = attention_fp4p_head(q8[i], sq[i], k8[i], sk[i], v8[i], qi["sv"], scale, causal, tile)
        outs.append(o)
        lses.append(l)
    O = np.stack(outs).reshape(lead + outs[0].shape)
    L = np.stack(lses).reshape(lead + lses[0].shape)
    return O, L, qi

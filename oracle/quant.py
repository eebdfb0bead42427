"""Quantisation emulation and the quantised-attention oracle.  TEST
INFRASTRUCTURE ONLY.

The quantised workload follows the token-level INT8 idea of [INT-FA post]
(section describing INT-FlashAttention: integer GEMMs for the scores, one
fp32 scale per token of Q and of K, post-training quantisation), with V in
OCP FP8 E4M3 under one per-tensor scale and the probabilities P cast to
E4M3 before the P.V product.  Steps, in order:

  1. per token (row of Q or K, in fp32): s = max|x| / 127 (fp32 division),
     q = clamp(rint(x / s), -127, 127) with rint = round half to even;
     a zero row gets s = 0 and q = 0;
  2. V per tensor: s_v = max|V| / 448 (fp32), codes = E4M3(V / s_v);
  3. S_int = Q8 K8^T accumulated exactly (int64 here; the GPU path's int32
     accumulator cannot overflow: |S_int| <= 127^2 * d);
  4. S = S_int * s_q[i] * s_k[j] * scale, in fp64; masked as in
     ``oracle.attention``;
  5. m = rowmax S, P = exp(S - m), l = rowsum P (unquantised P);
  6. P~ = E4M3(P); O = (P~ . (decode(codes) * s_v)) / l;  LSE = m + ln l.

E4M3 is OCP 8-bit floating point "E4M3FN": 1 sign, 4 exponent (bias 7), 3
mantissa bits, subnormals m * 2^-9, no infinities, 0x7F/0xFF are NaN, the
largest finite magnitude is 448.

Readings where the sources are silent:
  * all divisions are IEEE fp32, correctly rounded (numpy float32 '/');
  * E4M3 encoding rounds to nearest, ties to the even code, and saturates
    magnitudes >= 448 to 448 (the per-tensor scale maps max|V| to 448, so
    only rounding can push a value past it);
  * a negative value that rounds to zero keeps its sign (code 0x80);
  * P is cast with its running-max-free value exp(S - m_final) here; the
    kernel casts exp(S - m_running) (the difference is where E4M3 rounding
    lands, inside the quantised tolerance);
  * l sums the unquantised P: only the MFMA operand is cast.

All-INT8 variant (the [INT-FA post]'s INT8 GEMMs in place of the floating
point ones for both products of the attention): steps 1, 3, 4, 5 as above,
then
  2'. V per tensor in int8: s_v = max|V| / 127 (fp32), codes =
      clamp(rint(V / s_v), -127, 127); a zero tensor gets s_v = 0;
  6'. P8 = rint(127 P) in [0, 127] (P <= 1, its scale is the constant
      1/127); O = (P8 . V8) * s_v / (127 l); LSE = m + ln l.
Reading: P is quantised against the final row max here (the kernel raises
its running max on every increase, so its P also stays <= 1, and the two
differ only where the 1/127 rounding lands).

Parity status: the E4M3 table is pinned to the format's closed form and to
torch's float8_e4m3fn; encoding to exhaustive midpoint/tie sweeps and to
torch's cast; int8 per-token quantisation to torch.round; the exact integer
scores to a brute-force Python-int loop; the attention steps 4-6 reuse the
pinned definition's structure and are pinned by the uniform-score and
one-hot closed forms under quantisation (tests/test_oracle_pins.py); the
all-INT8 variant's per-tensor int8 to torch.round and its attention to the
uniform, two-key and one-hot closed forms (tests/test_oracle_variants.py).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN code (uint8) -> value (fp64); NaN codes -> nan."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# non-negative finite magnitudes in code order 0x00 .. 0x7E (monotonic)
_E4M3_TABLE = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Value -> E4M3FN code: round to nearest, ties to even, saturating at
    448.  ``x`` is taken exactly (fp32 or fp64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.signbit(x)
    t = _E4M3_TABLE
    hi = np.searchsorted(t, a, side="left")          # first t[hi] >= a
    hi = np.clip(hi, 1, len(t) - 1)
    lo = hi - 1
    mid = (t[lo] + t[hi]) * 0.5                        # exact (dyadic)
    code = np.where(a < mid, lo, np.where(a > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == 0.0, 0, code)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_per_token_int8(x32):
    """Symmetric per-token int8: x32 [..., d] fp32 -> (q8 int8, scale fp32 [...])."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    qf = (x32 / safe[..., None]).astype(np.float32)
    q8 = np.clip(np.rint(qf), -127, 127)
    q8 = np.where(s[..., None] > 0, q8, 0).astype(np.int8)
    return q8, s


def quantize_per_tensor_e4m3(x32):
    """Per-tensor E4M3: x32 fp32 (any shape) -> (codes uint8, scale fp32)."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    if s == 0:
        return np.zeros(x32.shape, np.uint8), s
    return e4m3_encode((x32 / s).astype(np.float32)), s


def quantize_per_tensor_int8(x32):
    """Per-tensor symmetric int8 (the all-INT8 variant's V): x32 fp32 (any
    shape) -> (q8 int8, scale fp32) with s = max|x| / 127 and
    q = clamp(rint(x / s), -127, 127) in fp32; a zero tensor gets s = 0."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s = np.float32(amax / np.float32(127.0))
    if s == 0:
        return np.zeros(x32.shape, np.int8), s
    return np.clip(np.rint((x32 / s).astype(np.float32)), -127, 127).astype(np.int8), s


def quantize_prob_int8(p) -> np.ndarray:
    """P in [0, 1] -> rint(127 P), round half to even (values 0 .. 127)."""
    return np.rint(127.0 * np.asarray(p, np.float64))


def qk_int(q8, k8) -> np.ndarray:
    """Exact integer scores Q8 K8^T for one head (int64)."""
    return np.asarray(q8, np.int64) @ np.asarray(k8, np.int64).T


def attention_q8_head(q8, sq, k8, sk, v_codes, sv, scale: float, causal: bool = False):
    """Steps 3-6 for one head from quantised inputs.  Returns (O, LSE) fp64."""
    Nq, Nk = q8.shape[0], k8.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    s = qk_int(q8, k8).astype(np.float64)
    s = s * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * float(scale)
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        s = np.where(j <= i + (Nk - Nq), s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    p_q = e4m3_decode(e4m3_encode(p))
    vq = e4m3_decode(v_codes) * float(sv)
    return (p_q @ vq) / l[:, None], m + np.log(l)


def quantize_inputs(q32, k32, v32):
    """Steps 1-2 on whole tensors [..., N, d] (fp32 values of the bf16
    inputs).  Returns dict(q8, sq, k8, sk, v8, sv)."""
    q8, sq = quantize_per_token_int8(q32)
    k8, sk = quantize_per_token_int8(k32)
    v8, sv = quantize_per_tensor_e4m3(v32)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv)


def attention_q8(q32, k32, v32, scale: float, causal: bool = False):
    """Whole quantised forward on [..., N, d] tensors.  Returns (O, LSE, quantised inputs)."""
    qi = quantize_inputs(q32, k32, v32)
    lead = np.asarray(q32).shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    shp = lambda a: a.reshape((n,) + a.shape[len(lead):])
    q8, sq, k8, sk, v8 = (shp(qi[x]) for x in ("q8", "sq", "k8", "sk", "v8"))
    outs, lses = [], []
    for i in range(n):
        o, l = attention_q8_head(q8[i], sq[i], k8[i], sk[i], v8[i], qi["sv"], scale, causal)
        outs.append(o)
        lses.append(l)
    O = np.stack(outs).reshape(lead + outs[0].shape)
    L = np.stack(lses).reshape(lead + lses[0].shape)
    return O, L, qi


def attention_i8_head(q8, sq, k8, sk, v8, sv, scale: float, causal: bool = False):
    """All-INT8 steps 3-5, 6' for one head from quantised inputs (v8 int8
    per-tensor).  Returns (O, LSE) fp64."""
    Nq, Nk = q8.shape[0], k8.shape[0]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    s = qk_int(q8, k8).astype(np.float64)
    s = s * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * float(scale)
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        s = np.where(j <= i + (Nk - Nq), s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = quantize_prob_int8(p) @ np.asarray(v8, np.float64)
    return o * (float(sv) / 127.0) / l[:, None], m + np.log(l)


def attention_i8(q32, k32, v32, scale: float, causal: bool = False):
    """Whole all-INT8 forward on [..., N, d] tensors.  Returns (O, LSE,
    quantised inputs dict(q8, sq, k8, sk, v8, sv))."""
    q8, sq = quantize_per_token_int8(q32)
    k8, sk = quantize_per_token_int8(k32)
    v8, sv = quantize_per_tensor_int8(v32)
    lead = np.asarray(q32).shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    shp = lambda a: a.reshape((n,) + a.shape[len(lead):])
    outs, lses = [], []
    for i in range(n):
        o, l = attention_i8_head(shp(q8)[i], shp(sq)[i], shp(k8)[i], shp(sk)[i], shp(v8)[i], sv, scale, causal)
        outs.append(o)
        lses.append(l)
    O = np.stack(outs).reshape(lead + outs[0].shape)
    L = np.stack(lses).reshape(lead + lses[0].shape)
    return O, L, dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv)

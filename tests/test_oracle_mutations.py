"""Planted mistakes in copies of the oracle must each fail at least one pin.

The copies below follow the oracle's steps with one switchable mistake each;
with no mistake switched on they must equal the oracle bit for bit, so the
pins are shown to catch the mistakes a reader would plausibly make in it:
a dropped term, a wrong sign or index, a transposed or swapped operand, a
wrong base or normaliser, an off-by-one mask, a wrong rounding rule.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as BW
from oracle import quant as Q
from oracle import recurrence as R
from tests import oracle_pins as P


def attn_variant(q, k, v, scale, causal, mistake=None):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    Nq, Nk = q.shape[0], k.shape[0]
    sc = {"drop_scale": 1.0, "sqrt_scale": math.sqrt(scale)}.get(mistake, scale)
    kk = k[::-1] if mistake == "reversed_keys_only" else k
    s = q @ kk.T * sc
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        vis = {"causal_strict": j < i + (Nk - Nq), "causal_top_left": j <= i}.get(mistake, j <= i + (Nk - Nq))
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(m[:, None] - s) if mistake == "exp_sign" else np.exp(s - m[:, None])
    l = e.sum(axis=1)
    vv = v[::-1] if mistake == "reversed_values" else v
    if mistake == "no_normalise":
        o = e @ vv
    elif mistake == "normalise_by_count":
        o = (e @ vv) / Nk
    else:
        o = (e @ vv) / l[:, None]
    lse = {"lse_no_max": np.log(l), "lse_log2": m + np.log2(l), "lse_plus_max": 2 * m + np.log(l)}.get(
        mistake, m + np.log(l))
    return o, lse


ATTN_MISTAKES = ["drop_scale", "sqrt_scale", "reversed_keys_only", "causal_strict", "causal_top_left",
                 "exp_sign", "reversed_values", "no_normalise", "normalise_by_count", "lse_no_max",
                 "lse_log2", "lse_plus_max"]


def _fails_some_pin(fn, pins):
    failed = []
    for pin in pins:
        try:
            pin(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_equals_oracle():
    rng = np.random.default_rng(7)
    for causal in (False, True):
        q, k, v = rng.standard_normal((5, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 3))
        o1, l1 = attn_variant(q, k, v, 0.5, causal)
        o2, l2 = A.attention_head(q, k, v, 0.5, causal)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("mistake", ATTN_MISTAKES)
def test_attention_mistake_is_caught(mistake):
    with np.errstate(all="ignore"):
        failed = _fails_some_pin(lambda q, k, v, s, c: attn_variant(q, k, v, s, c, mistake), P.ATTENTION_PINS)
    assert failed, f"no pin catches {mistake}"


def tiled_variant(q, k, v, scale, causal, rows_per_block=3, keys_per_block=2, mistake=None):
    """The recurrence of oracle.recurrence with one switchable mistake."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    Nq, Nk = q.shape[0], k.shape[0]
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
                block = np.where(keys[None, :] > qrows[:, None] + (Nk - Nq), -np.inf, block)
            bmax = block.max(axis=1)
            new_top = np.maximum(top, bmax)
            ref = np.where(np.isfinite(new_top), new_top, 0.0)
            history = np.exp(top - ref)
            if mistake == "history_not_rescaled":
                history = np.where(np.isfinite(top), 1.0, 0.0)
            wref = np.where(np.isfinite(bmax), bmax, 0.0) if mistake == "block_own_max" else ref
            weights = np.exp(block - wref[:, None])
            mass = (mass if mistake == "mass_not_rescaled" else mass * history) + weights.sum(axis=1)
            acc = acc * history[:, None] + weights @ v[keys]
            top = bmax if mistake == "max_not_running" else new_top
        out[qrows] = acc if mistake == "no_final_division" else acc / mass[:, None]
        lse[qrows] = top + np.log(mass)
    return out, lse


TILED_MISTAKES = ["history_not_rescaled", "mass_not_rescaled", "block_own_max", "no_final_division",
                  "max_not_running"]


def test_unmutated_tiled_copy_equals_oracle():
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((7, 4)), rng.standard_normal((11, 4)), rng.standard_normal((11, 3))
    for causal in (False, True):
        o1, l1 = tiled_variant(q, k, v, 0.5, causal)
        o2, l2 = R.online_forward(q, k, v, 0.5, causal, rows_per_block=3, keys_per_block=2)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("mistake", TILED_MISTAKES)
def test_recurrence_mistake_is_caught(mistake):
    with np.errstate(all="ignore"):
        failed = _fails_some_pin(lambda q, k, v, s, c: tiled_variant(q, k, v, s, c, mistake=mistake),
                                 P.ATTENTION_PINS)
    assert failed, f"no pin catches {mistake}"


# ------------------------------------------------------------ quantisation

def int8_variant(x32, mistake=None):
    x32 = np.asarray(x32, np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(128.0 if mistake == "divide_by_128" else 127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    qf = (x32 / safe[..., None]).astype(np.float32)
    if mistake == "floor":
        r = np.floor(qf)
    elif mistake == "half_away":
        r = np.sign(qf) * np.floor(np.abs(qf) + 0.5)
    elif mistake == "multiply_by_reciprocal":
        r = np.rint((x32 * (np.float32(1.0) / safe)[..., None]).astype(np.float32))
    else:
        r = np.rint(qf)
    q8 = np.where(s[..., None] > 0, np.clip(r, -127, 127), 0).astype(np.int8)
    return q8, s


def test_unmutated_int8_copy_equals_oracle():
    x = np.random.default_rng(9).standard_normal((30, 16)).astype(np.float32)
    a, sa = int8_variant(x)
    b, sb = Q.quantize_per_token_int8(x)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


@pytest.mark.parametrize("mistake", ["divide_by_128", "floor", "half_away", "multiply_by_reciprocal"])
def test_int8_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_int8_per_token(lambda x: int8_variant(x, mistake))


def e4m3_encode_variant(x, mistake):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    t = Q._E4M3_TABLE
    if mistake == "bias_8":
        t = t / 2.0
    hi = np.clip(np.searchsorted(t, a, side="left"), 1, len(t) - 1)
    lo = hi - 1
    mid = (t[lo] + t[hi]) * 0.5
    if mistake == "ties_away":
        tie = hi
    elif mistake == "ties_to_odd":
        tie = np.where(lo % 2 == 1, lo, hi)
    else:
        tie = np.where(lo % 2 == 0, lo, hi)
    code = np.where(a < mid, lo, np.where(a > mid, hi, tie))
    if mistake == "truncate":
        code = np.where(t[hi] == a, hi, lo)
    code = np.where(a == 0.0, 0, code)
    code = np.where(a >= 448.0, 0x7E, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def test_unmutated_e4m3_copy_equals_oracle():
    x = P._e4m3_sweep()
    assert np.array_equal(e4m3_encode_variant(x, None), Q.e4m3_encode(x))


@pytest.mark.parametrize("mistake", ["bias_8", "ties_away", "ties_to_odd", "truncate"])
def test_e4m3_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_e4m3_encode(lambda x: e4m3_encode_variant(x, mistake), Q.e4m3_decode)


def q8_attention_variant(q8, sq, k8, sk, v8, sv, scale, mistake=None):
    s = Q.qk_int(q8, k8).astype(np.float64) * np.asarray(sq, np.float64)[:, None] * \
        np.asarray(sk, np.float64)[None, :] * scale
    if mistake == "scale_q_twice":
        s = s * np.asarray(sq, np.float64)[:, None]
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    pq = p if mistake == "p_not_quantised" else Q.e4m3_decode(Q.e4m3_encode(p))
    l = pq.sum(axis=1) if mistake == "l_from_quantised_p" else p.sum(axis=1)
    svv = 1.0 if mistake == "v_scale_dropped" else float(sv)
    return (pq @ (Q.e4m3_decode(v8) * svv)) / l[:, None], m + np.log(l)


def test_unmutated_q8_copy_equals_oracle():
    rng = np.random.default_rng(10)
    q8 = rng.integers(-127, 128, (4, 16)).astype(np.int8)
    k8 = rng.integers(-127, 128, (6, 16)).astype(np.int8)
    v8 = rng.integers(0, 0x7E, (6, 8)).astype(np.uint8)
    sq, sk = rng.random(4).astype(np.float32) * 0.01, rng.random(6).astype(np.float32) * 0.01
    a = q8_attention_variant(q8, sq, k8, sk, v8, np.float32(0.5), 0.3)
    b = Q.attention_q8_head(q8, sq, k8, sk, v8, np.float32(0.5), 0.3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("mistake", ["scale_q_twice", "p_not_quantised", "l_from_quantised_p", "v_scale_dropped"])
def test_q8_attention_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_q8_attention(lambda *a: q8_attention_variant(*a, mistake=mistake), Q.e4m3_decode)


def bwd_variant(q, k, v, do, scale, causal, mistake=None):
    """The chain rule of oracle.backward with one switchable mistake."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    Nq, Nk = q.shape[0], k.shape[0]
    s = q @ k.T * scale
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        vis = {"causal_strict": j < i + (Nk - Nq), "causal_top_left": j <= i}.get(mistake, j <= i + (Nk - Nq))
        if mistake != "no_mask":
            s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    p = e / e.sum(axis=1)[:, None]
    dv = (e if mistake == "dv_unnormalised" else p).T @ do
    dp = do @ v.T
    if mistake == "drop_softmax_term":
        ds = p * dp
    elif mistake == "softmax_term_over_columns":
        ds = p * (dp - (p * dp).sum(axis=0)[None, :])
    elif mistake == "softmax_term_sign":
        ds = p * ((p * dp).sum(axis=1)[:, None] - dp)
    else:
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
    dq = (1.0 if mistake == "dq_no_scale" else scale) * (ds @ (v if mistake == "dq_uses_v" else k))
    dk = (1.0 if mistake == "dk_no_scale" else scale) * ((ds if mistake == "dk_untransposed_ds" else ds.T) @ q)
    return dq, dk, dv


BWD_MISTAKES = ["causal_strict", "causal_top_left", "no_mask", "dv_unnormalised", "drop_softmax_term",
                "softmax_term_over_columns", "softmax_term_sign", "dq_no_scale", "dq_uses_v", "dk_no_scale",
                "dk_untransposed_ds"]


def test_unmutated_backward_copy_equals_oracle():
    rng = np.random.default_rng(9)
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((5, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 3)),
                       rng.standard_normal((5, 3)))
        for a, b in zip(bwd_variant(q, k, v, do, 0.5, causal), BW.attention_backward_head(q, k, v, do, 0.5, causal)):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("mistake", BWD_MISTAKES)
def test_backward_mistake_is_caught(mistake):
    fwd = lambda q, k, v, s, c: A.attention_head(q, k, v, s, c)
    fd = lambda fn: P.pin_bwd_finite_difference(fn, fwd)
    fd.__name__ = "pin_bwd_finite_difference"
    with np.errstate(all="ignore"):
        failed = _fails_some_pin(lambda q, k, v, do, s, c: bwd_variant(q, k, v, do, s, c, mistake),
                                 P.BACKWARD_PINS + [fd])
    assert failed, f"no pin catches {mistake}"

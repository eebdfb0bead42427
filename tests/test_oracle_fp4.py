"""The MXFP4-P oracle against its pins, and planted mistakes in copies of it
(no GPU)."""
import numpy as np
import pytest

from oracle import fp4 as F4
from oracle import quant as Q
from oracle import rotated as RT
from tests import oracle_pins as P


def test_e2m1_pin():
    P.pin_e2m1(F4.e2m1_encode, F4.e2m1_decode)


def test_mx_p_pin():
    P.pin_mx_p(F4.quantize_p_mx, F4.e2m1_encode, F4.e2m1_decode)


def test_fp4p_attention_pin():
    P.pin_fp4p_attention(F4.attention_fp4p_head, RT.attention_fp8_head)


def test_fp4p_recurrence_pin():
    P.pin_fp4p_recurrence(F4.attention_fp4p_head)


def test_recurrence_without_rescale_is_caught():
    """A recurrence that forgets to rescale the accumulated O and l when the
    running max rises fails the recurrence pin."""
    def no_rescale(q8, sq, k8, sk, v8, sv, scale, causal=False, tile=64, quantize=None):
        s = Q.e4m3_decode(q8) @ Q.e4m3_decode(k8).T * sq[:, None] * sk[None, :] * scale
        if causal:
            Nq, Nk = s.shape
            s = np.where(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + Nk - Nq, s, -np.inf)
        vd = Q.e4m3_decode(v8) * float(sv)
        m = np.full(s.shape[0], -np.inf)
        l = np.zeros(s.shape[0])
        acc = np.zeros((s.shape[0], vd.shape[1]))
        for t0 in range(0, s.shape[1], tile):
            st = s[:, t0:t0 + tile]
            m = np.maximum(m, st.max(axis=1))
            p = np.exp(st - m[:, None])
            l = l + p.sum(axis=1)
            acc = acc + quantize(p) @ vd[t0:t0 + tile]
        return acc / l[:, None], m + np.log(l)
    with pytest.raises(AssertionError):
        P.pin_fp4p_recurrence(no_rescale)


def test_whole_forward_runs_per_head():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((2, 40, 128)).astype(np.float32) for _ in range(3))
    O, L, qi = F4.attention_fp4p(q, k, v, None, 128 ** -0.5, True)
    o1, l1 = F4.attention_fp4p_head(qi["q8"][1], qi["sq"][1], qi["k8"][1], qi["sk"][1], qi["v8"][1], qi["sv"],
                                    128 ** -0.5, True)
    assert np.array_equal(O[1], o1) and np.array_equal(L[1], l1)


# ---- planted mistakes

def encode_trunc(x):
    x = np.asarray(x, np.float64)
    t = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    code = np.clip(np.searchsorted(t, np.abs(x), side="right") - 1, 0, 7)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def encode_ties_up(x):
    x = np.asarray(x, np.float64)
    t = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.abs(x)
    hi = np.clip(np.searchsorted(t, a, side="left"), 1, 7)
    lo = hi - 1
    code = np.where(a < (t[lo] + t[hi]) / 2, lo, hi)
    code = np.where(a >= 6, 7, np.where(a == 0, 0, code))
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


@pytest.mark.parametrize("enc", [encode_trunc, encode_ties_up], ids=["truncate", "ties_up"])
def test_e2m1_mistake_is_caught(enc):
    with pytest.raises(AssertionError):
        P.pin_e2m1(enc, F4.e2m1_decode)


def mx_variant(p, block=32, mistake=None):
    p = np.asarray(p, np.float64)
    Nq, Nk = p.shape
    blk = 16 if mistake == "block_16" else block
    nb = -(-Nk // blk)
    pp = np.zeros((Nq, nb * blk))
    pp[:, :Nk] = p
    pb = pp.reshape(Nq, nb, blk)
    pmax = pb.max(axis=2) if mistake != "row_scale" else np.repeat(pp.max(axis=1, keepdims=True), nb, axis=1)
    _, E = np.frexp(np.where(pmax > 0, pmax, 1.0))
    e = (E - 1 - (1 if mistake == "emax_1" else 2)).astype(np.float64)
    y = pb / np.exp2(e)[:, :, None]
    out = F4.e2m1_decode(F4.e2m1_encode(y)) * np.exp2(e)[:, :, None]
    out = np.where((pmax > 0)[:, :, None], out, 0.0)
    return out.reshape(Nq, nb * blk)[:, :Nk]


def test_unmutated_mx_copy_equals_oracle():
    p = np.random.default_rng(4).random((3, 77)) ** 3
    assert np.array_equal(mx_variant(p), F4.quantize_p_mx(p))


@pytest.mark.parametrize("mistake", ["block_16", "row_scale", "emax_1"])
def test_mx_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_mx_p(lambda p: mx_variant(p, mistake=mistake), F4.e2m1_encode, F4.e2m1_decode)


def attn_variant(q8, sq, k8, sk, v8, sv, scale, causal=False, mistake=None):
    # one tile (the whole row) is enough for the closed-form pins
    s = Q.e4m3_decode(q8) @ Q.e4m3_decode(k8).T
    s = s * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * float(scale)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    pq = F4.quantize_p_mx(p)
    l = pq.sum(axis=1) if mistake == "l_of_quantised_p" else p.sum(axis=1)
    vd = Q.e4m3_decode(v8) * (1.0 if mistake == "no_v_scale" else float(sv))
    return (pq @ vd) / l[:, None], m + np.log(l)


def test_unmutated_attn_copy_equals_oracle_on_one_tile():
    rng = np.random.default_rng(8)
    q8, k8, v8 = (Q.e4m3_encode(rng.standard_normal((n, 16)) * 30) for n in (5, 40, 40))
    sq, sk = np.full(5, 0.05, np.float32), np.full(40, 0.04, np.float32)
    a = attn_variant(q8, sq, k8, sk, v8, np.float32(0.1), 0.3)
    b = F4.attention_fp4p_head(q8, sq, k8, sk, v8, np.float32(0.1), 0.3, False, 40)
    assert np.allclose(a[0], b[0], atol=1e-14, rtol=0) and np.allclose(a[1], b[1], atol=1e-14)


@pytest.mark.parametrize("mistake", ["l_of_quantised_p", "no_v_scale"])
def test_fp4p_attention_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_fp4p_attention(lambda *a, **kw: attn_variant(*a, **kw, mistake=mistake), RT.attention_fp8_head)

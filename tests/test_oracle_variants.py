"""GQA and packed variable-length oracles against their pins, and planted
mistakes in copies of them (no GPU)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import variants as V
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.GQA_PINS, ids=lambda f: f.__name__)
def test_gqa_pins(pin):
    pin(V.attention_gqa)


@pytest.mark.parametrize("pin", P.VARLEN_PINS, ids=lambda f: f.__name__)
def test_varlen_pins(pin):
    pin(V.attention_varlen)


def test_gqa_backward_pin():
    P.pin_gqa_backward_torch(V.attention_backward_gqa)


def test_varlen_backward_pin():
    P.pin_varlen_backward(V.attention_backward_varlen, V.attention_varlen)


def test_varlen_backward_mistake_is_caught():
    """Gradients of the no-key rows left to the dense formula (NaN/garbage) or a
    shared head's dK not summed over its query heads must fail the pin."""
    def no_sum(q, k, v, do, cq, ck, s, c):
        dq, dk, dv = V.attention_backward_varlen(q, k, v, do, cq, ck, s, c)
        return dq, dk / 2.0, dv
    with pytest.raises(AssertionError):
        P.pin_varlen_backward(no_sum, V.attention_varlen)


def test_kv_head_rejects_uneven_groups():
    with pytest.raises(ValueError):
        V.kv_head(0, 6, 4)


# ---- planted mistakes: each must fail a pin
def gqa_variant(q, k, v, scale, causal, mistake=None):
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    O = np.empty(q.shape[:3] + (v.shape[3],))
    L = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            g = h % Hkv if mistake == "interleaved_heads" else h // (H // Hkv)
            O[b, h], L[b, h] = A.attention_head(q[b, h], k[b, g], v[b, g], scale, causal)
    return O, L


def varlen_variant(q, k, v, cu_q, cu_k, scale, causal, mistake=None):
    H, Hkv = q.shape[0], k.shape[0]
    O = np.zeros(q.shape[:2] + (v.shape[2],))
    L = np.full(q.shape[:2], -np.inf)
    for s in range(len(cu_q) - 1):
        qa, qb = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        if mistake == "keys_one_short":
            kb = max(ka, kb - 1)
        for h in range(H):
            g = h // (H // Hkv)
            Nq, Nk = qb - qa, kb - ka
            if Nq == 0 or Nk == 0:
                continue
            if mistake == "top_left_causal":
                qq, kk, vv = q[h, qa:qb], k[g, ka:kb], v[g, ka:kb]
                s_ = qq @ kk.T * scale
                if causal:
                    s_ = np.where(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None], s_, -np.inf)
                m = s_.max(axis=1)
                e = np.exp(s_ - m[:, None])
                O[h, qa:qb], L[h, qa:qb] = (e @ vv) / e.sum(1)[:, None], m + np.log(e.sum(1))
                continue
            O[h, qa:qb], L[h, qa:qb] = V._seq_attention(q[h, qa:qb], k[g, ka:kb], v[g, ka:kb], scale, causal)
    return O, L


def test_unmutated_variant_copies_equal_oracle():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((2, 4, 5, 3)), rng.standard_normal((2, 2, 7, 3)), rng.standard_normal((2, 2, 7, 3))
    for a, b in zip(gqa_variant(q, k, v, 0.5, True), V.attention_gqa(q, k, v, 0.5, True)):
        assert np.array_equal(a, b)
    cq, ck = np.array([0, 3, 7]), np.array([0, 4, 9])
    q, k, v = rng.standard_normal((2, 7, 3)), rng.standard_normal((1, 9, 3)), rng.standard_normal((1, 9, 3))
    for a, b in zip(varlen_variant(q, k, v, cq, ck, 0.5, True), V.attention_varlen(q, k, v, cq, ck, 0.5, True)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mistake", ["interleaved_heads"])
def test_gqa_mistake_is_caught(mistake):
    failed = []
    for pin in P.GQA_PINS:
        try:
            pin(lambda q, k, v, s, c: gqa_variant(q, k, v, s, c, mistake))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed


@pytest.mark.parametrize("mistake", ["keys_one_short", "top_left_causal"])
def test_varlen_mistake_is_caught(mistake):
    failed = []
    for pin in P.VARLEN_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda q, k, v, cq, ck, s, c: varlen_variant(q, k, v, cq, ck, s, c, mistake))
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed


# ---- all-INT8 quantised variant
from oracle import quant as Q


def test_int8_per_tensor_pin():
    P.pin_int8_per_tensor(Q.quantize_per_tensor_int8)


def test_i8_attention_pin():
    P.pin_i8_attention(Q.attention_i8_head)


def i8_variant(q8, sq, k8, sk, v8, sv, scale, causal=False, mistake=None):
    s = Q.qk_int(q8, k8).astype(np.float64) * sq[:, None].astype(np.float64) * sk[None, :].astype(np.float64) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    p8 = {"floor_p": np.floor(127 * p), "scale_128": np.rint(128 * p)}.get(mistake, np.rint(127 * p))
    div = 1.0 if mistake == "no_127" else 127.0
    o = p8 @ v8.astype(np.float64) * (float(sv) / div)
    return (o if mistake == "no_normalise" else o / l[:, None]), m + np.log(l)


def test_unmutated_i8_copy_equals_oracle():
    rng = np.random.default_rng(11)
    q8 = rng.integers(-127, 128, (5, 8)).astype(np.int8)
    k8 = rng.integers(-127, 128, (7, 8)).astype(np.int8)
    v8 = rng.integers(-127, 128, (7, 8)).astype(np.int8)
    sq, sk = np.full(5, 0.01, np.float32), np.full(7, 0.02, np.float32)
    for a, b in zip(i8_variant(q8, sq, k8, sk, v8, np.float32(0.3), 0.5),
                    Q.attention_i8_head(q8, sq, k8, sk, v8, np.float32(0.3), 0.5)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mistake", ["floor_p", "scale_128", "no_127", "no_normalise"])
def test_i8_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_i8_attention(lambda *a, **kw: i8_variant(*a, **kw, mistake=mistake))


def test_int8_per_tensor_mistake_is_caught():
    def floor_q(x):
        x = np.asarray(x, np.float32)
        s = np.float32(np.float32(np.max(np.abs(x))) / np.float32(127.0)) if x.size else np.float32(0)
        if s == 0:
            return np.zeros(x.shape, np.int8), s
        return np.clip(np.floor(x / s), -127, 127).astype(np.int8), s
    with pytest.raises(AssertionError):
        P.pin_int8_per_tensor(floor_q)


def test_prob_int8_rounding_pin():
    """P8 = rint(127 P): brute force against Python's round (half to even) on
    probabilities whose 127 P are exact halves and on random ones; the range
    is 0 .. 127 with P = 1 at 127."""
    halves = np.arange(0, 255) / 2.0          # 127 P = 0, 0.5, ..., 127
    p = halves / 127.0
    exact = 127.0 * p == halves               # keep the ties that survive the division
    got = Q.quantize_prob_int8(p)
    want = np.array([round(float(x)) for x in 127.0 * p])
    assert np.array_equal(got, want)
    assert exact.sum() > 100 and np.array_equal(got[exact], [round(x) for x in halves[exact]])
    assert got[exact][1] == 0 and got[exact][3] == 2   # 0.5 -> 0, 1.5 -> 2
    r = np.random.default_rng(3).random(1000)
    assert np.array_equal(Q.quantize_prob_int8(r), [round(127.0 * x) for x in r])
    assert Q.quantize_prob_int8(np.array([0.0, 1.0])).tolist() == [0.0, 127.0]


def test_i8_whole_tensor_pin():
    """The all-INT8 forward on [B, H, N, d] tensors, from unquantised inputs:
    (a) Q = 0 gives uniform P (P8 = 127 on every key), so each head's O is
    s_v times the mean of its own V8 rows and LSE = ln Nk; V differs per
    head, so a head taking another head's K/V fails; (b) orthogonal keys and
    a query aligned with one key at a large score select that key's V8 row;
    V8 and s_v are the per-tensor int8 codes of V (within s_v / 2 of V)."""
    rng = np.random.default_rng(21)
    B, H, Nq, Nk, d = 2, 3, 4, 6, 8
    v = rng.standard_normal((B, H, Nk, d)).astype(np.float32) + np.arange(B * H).reshape(B, H, 1, 1)
    k = rng.standard_normal((B, H, Nk, d)).astype(np.float32)
    O, L, qi = Q.attention_i8(np.zeros((B, H, Nq, d), np.float32), k, v, 0.5)
    assert O.shape == (B, H, Nq, d) and L.shape == (B, H, Nq)
    sv = float(qi["sv"])
    assert abs(sv - float(np.max(np.abs(v))) / 127.0) <= 1e-6 * sv
    assert np.max(np.abs(qi["v8"] * sv - v)) <= 0.5 * sv * (1 + 1e-6)
    for b in range(B):
        for h in range(H):
            want = sv * qi["v8"][b, h].astype(np.float64).mean(axis=0)
            assert np.max(np.abs(O[b, h] - want)) <= 1e-12
    assert np.max(np.abs(L - np.log(Nk))) <= 1e-12
    # (b): key j = e_j * 4, query i aligned with key i; scores 4 * 4 * scale apart
    k = np.zeros((1, 1, Nk, d), np.float32)
    k[0, 0, np.arange(Nk), np.arange(Nk)] = 4.0
    q = np.zeros((1, 1, Nq, d), np.float32)
    q[0, 0, np.arange(Nq), np.arange(Nq)] = 4.0
    v1 = v[:1, :1]
    O, _, qi = Q.attention_i8(q, k, v1, 4.0)   # exp(-64) below 127's rounding: P8 one-hot
    for i in range(Nq):
        assert np.max(np.abs(O[0, 0, i] - float(qi["sv"]) * qi["v8"][0, 0, i])) <= 1e-12

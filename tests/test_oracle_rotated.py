"""The rotated FP8 oracle against its pins, and planted mistakes in copies of
it (no GPU)."""
import numpy as np
import pytest

from oracle import quant as Q
from oracle import rotated as R
from tests import oracle_pins as P


def test_hadamard_pin():
    P.pin_hadamard(R.hadamard)


def test_fwht_pin():
    P.pin_fwht(R.fwht_f32, R.hadamard)


def test_rotate_quantize_pin():
    P.pin_rotate_quantize(R.rotate_quantize_e4m3)


def test_fp8_attention_pin():
    P.pin_fp8_attention(R.attention_fp8_head)


def test_rotation_lowers_error_pin():
    P.pin_rotation_lowers_error(R.attention_rotated_fp8)


def test_rejects():
    with pytest.raises(ValueError):
        R.hadamard(96)
    with pytest.raises(ValueError):
        R.rotate_quantize_e4m3(np.zeros((4, 8), np.float32), np.ones(4), 2)
    with pytest.raises(ValueError):
        R.rotate_quantize_e4m3(np.zeros((4, 8), np.float32), np.full(8, 0.5), 2)


# ---- planted mistakes: each must fail at least one pin

def fwht_variant(x, mistake):
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        lo, hi = z[..., 0, :].copy(), z[..., 1, :].copy()
        z[..., 0, :] = lo + hi
        z[..., 1, :] = (hi - lo) if mistake == "flipped_butterfly" else (lo - hi)
        y = z.reshape(lead + (d,))
        h *= 2 if mistake != "skip_stride" or h != 4 else 4
    return y


@pytest.mark.parametrize("mistake", ["flipped_butterfly", "skip_stride"])
def test_fwht_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_fwht(lambda x: fwht_variant(x, mistake), R.hadamard)


def rq_variant(x32, signs, block_rows, mistake):
    x32 = np.asarray(x32, np.float32)
    N, d = x32.shape[-2:]
    if signs is None:
        y, post = x32, None
    else:
        y = R.fwht_f32(x32 if mistake == "signs_ignored" else x32 * np.asarray(signs, np.float32))
        post = None if mistake == "no_normalisation" else np.float32(1.0 / np.sqrt(d))
    codes = np.zeros(y.shape, np.uint8)
    scales = np.zeros(y.shape[:-1], np.float32)
    whole = np.max(np.abs(y), axis=(-2, -1)).astype(np.float32)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        blk = y[..., r0:r1, :]
        amax = whole if mistake == "per_tensor_scale" else np.max(np.abs(blk), axis=(-2, -1)).astype(np.float32)
        div = np.float32(240.0 if mistake == "wrong_max" else 448.0)
        sc = (amax / div).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1)).astype(np.float32)
        c = Q.e4m3_encode((blk / safe[..., None, None]).astype(np.float32))
        codes[..., r0:r1, :] = np.where((sc > 0)[..., None, None], c, 0)
        rs = sc if post is None else (sc * post).astype(np.float32)
        scales[..., r0:r1] = rs[..., None]
    return codes, scales


def test_unmutated_rq_copy_equals_oracle():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 70, 128)).astype(np.float32)
    s = rng.choice([-1.0, 1.0], 128)
    for sg in (None, s):
        a, b = rq_variant(x, sg, 32, None), R.rotate_quantize_e4m3(x, sg, 32)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("mistake", ["signs_ignored", "no_normalisation", "per_tensor_scale", "wrong_max"])
def test_rotate_quantize_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_rotate_quantize(lambda x, s, b: rq_variant(x, s, b, mistake))


def attn_variant(q8, sq, k8, sk, v8, sv, scale, causal=False, mistake=None):
    s = Q.e4m3_decode(q8) @ Q.e4m3_decode(k8).T
    s = s * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * float(scale)
    Nq, Nk = s.shape
    if causal:
        i, j = np.arange(Nq)[:, None], np.arange(Nk)[None, :]
        s = np.where(j <= i + (0 if mistake == "top_left" else Nk - Nq), s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    pq = p if mistake == "p_unquantised" else Q.e4m3_decode(Q.e4m3_encode(p))
    if mistake == "l_of_quantised_p":
        l = pq.sum(axis=1)
    return (pq @ (Q.e4m3_decode(v8) * float(sv))) / l[:, None], m + np.log(l)


def test_unmutated_attn_copy_equals_oracle():
    rng = np.random.default_rng(6)
    q8, k8, v8 = (Q.e4m3_encode(rng.standard_normal((n, 16)) * 30) for n in (5, 7, 7))
    sq, sk = np.full(5, 0.05, np.float32), np.full(7, 0.04, np.float32)
    for causal in (False, True):
        a = attn_variant(q8, sq, k8, sk, v8, np.float32(0.1), 0.3, causal)
        b = R.attention_fp8_head(q8, sq, k8, sk, v8, np.float32(0.1), 0.3, causal)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("mistake", ["top_left", "p_unquantised", "l_of_quantised_p"])
def test_fp8_attention_mistake_is_caught(mistake):
    with pytest.raises(AssertionError):
        P.pin_fp8_attention(lambda *a, **kw: attn_variant(*a, **kw, mistake=mistake))


def test_rotation_of_q_only_is_caught():
    """Rotating Q but not K breaks Q K^T: the method's error claim fails."""
    def q_only(q, k, v, signs, scale, causal, block_rows):
        qi = R.quantize_inputs(q, k, v, signs, block_rows)
        if signs is not None:
            qi["k8"], qi["sk"] = R.rotate_quantize_e4m3(k, None, block_rows)
        o, l = R.attention_fp8_head(qi["q8"], qi["sq"], qi["k8"], qi["sk"], qi["v8"], qi["sv"], scale, causal)
        return o, l, qi
    with pytest.raises(AssertionError):
        P.pin_rotation_lowers_error(q_only)

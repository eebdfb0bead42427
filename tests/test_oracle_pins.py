"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import quant as Q
from oracle import recurrence as R
from tests import oracle_pins as P


def _definition(q, k, v, scale, causal):
    return A.attention_head(q, k, v, scale, causal, row_chunk=3)


def _tiled(q, k, v, scale, causal):
    return R.online_forward(q, k, v, scale, causal, rows_per_block=3, keys_per_block=2)


@pytest.mark.parametrize("pin", P.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_definition_pins(pin):
    pin(_definition)


@pytest.mark.parametrize("pin", P.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_recurrence_pins(pin):
    pin(_tiled)


def test_batched_equals_per_head():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((2, 3, 5, 4)), rng.standard_normal((2, 3, 9, 4)), rng.standard_normal((2, 3, 9, 4))
    O, L = A.attention(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            o, l = A.attention_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            assert np.array_equal(O[b, h], o) and np.array_equal(L[b, h], l)


def test_rows_sampler_matches_whole():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((11, 4)), rng.standard_normal((17, 4)), rng.standard_normal((17, 3))
    O, L = A.attention_head(q, k, v, 0.5, True)
    rows = [0, 4, 10]
    o, l = A.attention_rows(q, k, v, rows, 0.5, True)
    assert np.max(np.abs(o - O[rows])) <= 1e-14 and np.max(np.abs(l - L[rows])) <= 1e-14


def test_causal_rejects_more_queries_than_keys():
    with pytest.raises(ValueError):
        A.attention_head(np.zeros((5, 2)), np.zeros((4, 2)), np.zeros((4, 2)), 1.0, True)


def test_softmax_rows_pin():
    P.pin_rows_sum_to_one(A.softmax_rows)


def test_recurrence_equals_definition():
    P.pin_recurrence_equals_definition(R.online_forward,
                                       lambda q, k, v, s, c: A.attention_head(q, k, v, s, c))


def test_merge_pin():
    P.pin_merge(R.merge_states, lambda q, k, v, s, c: A.attention_head(q, k, v, s, c))


def test_split_kv_forward():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    O, L = A.attention_head(q, k, v, 0.3)
    O2, L2 = R.split_kv_forward(q, k, v, 0.3, [0, 7, 8, 33, 40],
                                lambda a, b, c, s: A.attention_head(a, b, c, s))
    assert np.max(np.abs(O - O2)) <= 1e-13 and np.max(np.abs(L - L2)) <= 1e-13


def test_e4m3_decode_pin():
    P.pin_e4m3_decode(Q.e4m3_decode)


def test_e4m3_encode_pin():
    P.pin_e4m3_encode(Q.e4m3_encode, Q.e4m3_decode)


def test_int8_per_token_pin():
    P.pin_int8_per_token(Q.quantize_per_token_int8)


def test_qk_int_pin():
    P.pin_qk_int(Q.qk_int)


def test_q8_attention_pin():
    P.pin_q8_attention(lambda q8, sq, k8, sk, v8, sv, sc: Q.attention_q8_head(q8, sq, k8, sk, v8, sv, sc),
                       Q.e4m3_decode)


def test_q8_int32_accumulator_bound():
    """|S_int| <= 127^2 * d fits int32 and is exact in fp32 for d <= 1024."""
    q8 = np.full((1, 128), 127, np.int8)
    k8 = np.full((1, 128), -127, np.int8)
    s = Q.qk_int(q8, k8)
    assert s[0, 0] == -127 * 127 * 128
    assert abs(int(s[0, 0])) < 2 ** 24 and float(np.float32(s[0, 0])) == float(s[0, 0])


def test_per_tensor_e4m3_maps_amax_to_448():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 50, 8)).astype(np.float32)
    codes, s = Q.quantize_per_tensor_e4m3(x)
    assert s == np.float32(np.abs(x).max() / np.float32(448))
    dec = Q.e4m3_decode(codes)
    assert np.nanmax(np.abs(dec)) == 448.0
    # relative error of E4M3 (3 mantissa bits) is at most 2^-4 above the subnormal range
    big = np.abs(x / s) >= 2.0 ** -6
    assert np.max(np.abs(dec[big] * s - x[big]) / np.abs(x[big])) <= 2.0 ** -4


def test_q8_oracle_close_to_fp64_definition():
    """Quantisation moves O only by a few percent on N(0,1) data (sanity,
    not a pin)."""
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 64, 128)).astype(np.float32) for _ in range(3))
    O, L, _ = Q.attention_q8(q, k, v, 128 ** -0.5)
    O2, L2 = A.attention(q, k, v, 128 ** -0.5)
    assert np.max(np.abs(O - O2)) < 0.1 and np.max(np.abs(L - L2)) < 0.1

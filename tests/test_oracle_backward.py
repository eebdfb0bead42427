"""The backward oracle against its pins (no GPU)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as BW
from tests import oracle_pins as P


def _bwd(q, k, v, do, scale, causal):
    return BW.attention_backward_head(q, k, v, do, scale, causal, row_chunk=2)


def _fwd(q, k, v, scale, causal):
    return A.attention_head(q, k, v, scale, causal)


@pytest.mark.parametrize("pin", P.BACKWARD_PINS, ids=lambda f: f.__name__)
def test_backward_pins(pin):
    pin(_bwd)


def test_backward_finite_difference():
    P.pin_bwd_finite_difference(_bwd, _fwd)


def test_backward_batched_equals_per_head():
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((2, 2, 5, 3)), rng.standard_normal((2, 2, 8, 3)),
                   rng.standard_normal((2, 2, 8, 3)), rng.standard_normal((2, 2, 5, 3)))
    got = BW.attention_backward(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(2):
            want = BW.attention_backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            for g, w in zip(got, want):
                assert np.array_equal(g[b, h], w)


def test_backward_causal_rejects_more_queries_than_keys():
    with pytest.raises(ValueError):
        BW.attention_backward_head(np.zeros((5, 2)), np.zeros((4, 2)), np.zeros((4, 2)), np.zeros((5, 2)), 1.0, True)

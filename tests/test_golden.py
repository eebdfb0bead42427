"""The oracle against hand-derived closed forms in tests/golden/ (no GPU)."""
import json
import os

import mpmath
import numpy as np
import pytest

from oracle import attention as A
from oracle import quant as Q
from oracle import recurrence as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _ev(expr):
    mpmath.mp.dps = 40
    env = {"e": mpmath.e, "ln": mpmath.log, "exp": mpmath.exp, "sqrt": mpmath.sqrt}
    return float(eval(expr.replace("^", "**"), {"__builtins__": {}}, env))


@pytest.mark.parametrize("case", GOLD["attention"], ids=lambda c: c["name"])
def test_attention_closed_forms(case):
    q, k, v = (np.array(case[x], np.float64) for x in ("q", "k", "v"))
    O_exp = np.array([[_ev(x) for x in row] for row in case["O"]])
    L_exp = np.array([_ev(x) for x in case["LSE"]])
    for fn in (lambda: A.attention_head(q, k, v, case["scale"], case["causal"]),
               lambda: R.online_forward(q, k, v, case["scale"], case["causal"], rows_per_block=1,
                                        keys_per_block=2)):
        O, L = fn()
        assert np.max(np.abs(O - O_exp)) <= 1e-14
        assert np.max(np.abs(L - L_exp)) <= 1e-14


@pytest.mark.parametrize("case", GOLD["int8_per_token"], ids=lambda c: str(c["row"]))
def test_int8_closed_forms(case):
    q8, s = Q.quantize_per_token_int8(np.array([case["row"]], np.float32))
    assert float(s[0]) == _ev(case["scale"])
    assert list(q8[0]) == case["q"]


@pytest.mark.parametrize("case", GOLD["e4m3"], ids=lambda c: c["x"])
def test_e4m3_closed_forms(case):
    x = _ev(case["x"])
    assert int(Q.e4m3_encode(np.array([x]))[0]) == case["code"]
    if abs(x) <= 448 and case["code"] not in (0,):
        # decoding the code gives the nearest representable value
        d = Q.e4m3_decode(np.array([case["code"]], np.uint8))[0]
        assert abs(d - x) <= abs(x) * 2.0 ** -4 or abs(x) < 2.0 ** -6

"""The polynomial exp2 of the software-exp2 split (csrc/prefill.hip,
exp2_poly), checked on the CPU against the mathematics.

* Its fp32 coefficients are those of the Remez fit.
* The fit equioscillates within 7.5e-5 relative error on [0, 1].
* The kernel's evaluation steps, emulated in fp32, stay within that bound
  (plus fp32 rounding) of the exact 2^x from -125 up to 128 (the softmax
  accepts tiles whose probabilities stay at or below 2^14; larger arguments
  only have to be large enough for its overflow check), integers and their
  neighbours included.  Arguments below -125, and -inf (masked keys), give
  0; arguments from 128 up give +inf.
A planted sign error in the range reduction breaks the bound."""
import os
import re

import numpy as np

from flashattention_forward_amd import exp2_poly_fit as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BOUND = 7.6e-5  # the fit's 7.48e-5 plus fp32 evaluation


def source_coefficients() -> np.ndarray:
    src = open(os.path.join(ROOT, "flashattention_forward_amd", "csrc", "prefill.hip")).read()
    num = r"([0-9.eE+-]+)f"
    m = re.search(r"kExp2C0 = " + num + r", kExp2C1 = " + num + r", kExp2C2 = " + num + r",\s*kExp2C3 = " + num, src)
    assert m, "exp2 polynomial constants not found"
    return np.array([float(x) for x in m.groups()], np.float32)


def _fma32(a, b, c):
    """fp32 fused multiply-add (the product of two fp32 values is exact in fp64)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def emulate(x, c=None, flip=False):
    """The kernel's steps in fp32: clamp, floor, fraction, Horner cubic, exponent add."""
    c = source_coefficients() if c is None else c
    x = np.asarray(x, np.float32)
    xc = np.maximum(x, np.float32(-125.0))
    n = np.floor(xc).astype(np.float32)
    with np.errstate(invalid="ignore"):  # x = +inf gives inf - inf here; the select below returns inf
        f = (n - xc if flip else xc - n).astype(np.float32)
    k = lambda v: np.full(f.shape, v, np.float32)
    p = _fma32(_fma32(_fma32(k(c[3]), f, k(c[2])), f, k(c[1])), f, k(c[0]))
    r = (p.view(np.int32) + (np.minimum(n, 127).astype(np.int32) << 23)).view(np.float32)
    return np.where(x < -125.0, np.float32(0.0), np.where(x >= 128.0, np.float32(np.inf), r))


def grid():
    rng = np.random.default_rng(7)
    ints = np.arange(-125, 128, dtype=np.float32)
    near = np.concatenate([np.nextafter(ints, np.float32(-np.inf)), np.nextafter(ints, np.float32(np.inf))])
    dense = np.linspace(-125.0, 16.0, 1_000_001, dtype=np.float32)
    rand = rng.uniform(-125.0, 128.0, 500_000).astype(np.float32)
    x = np.concatenate([ints, near, dense, rand, [np.nextafter(np.float32(128.0), np.float32(0.0))]])
    return x[(x >= -125.0) & (x < 128.0)]


def rel_err(y, x):
    exact = np.exp2(x.astype(np.float64))
    return np.abs(y.astype(np.float64) / exact - 1.0)


def test_coefficients_are_the_fit():
    assert np.array_equal(P.coefficients_f32(), source_coefficients())


def test_fit_equioscillates_within_bound():
    c, e = P.fit()
    assert 7.4e-5 < e < 7.5e-5
    g = np.linspace(0.0, 1.0, 100001)
    err = np.polyval(c[::-1], g) / 2.0 ** g - 1.0
    # degree + 2 = 5 extrema (the end points and three interior ones) reach the
    # bound with alternating signs
    d = np.diff(err)
    ext = [0] + [i for i in range(1, len(g) - 1) if d[i - 1] * d[i] <= 0] + [len(g) - 1]
    peaks = [np.sign(err[i]) for i in ext if abs(err[i]) > 0.999 * e]
    assert len(peaks) == 5 and all(peaks[i] != peaks[i + 1] for i in range(4))


def test_kernel_steps_within_bound():
    x = grid()
    y = emulate(x)
    assert np.all(np.isfinite(y)) and np.all(y > 0)
    assert rel_err(y, x).max() <= BOUND


def test_underflow_and_masked_keys_give_zero():
    x = np.array([-125.5, -126.0, -200.0, -1e30, -np.inf], np.float32)
    assert np.all(emulate(x) == 0.0)
    # 2^-125 itself is kept
    assert abs(float(emulate(np.array([-125.0], np.float32))[0]) / 2.0 ** -125 - 1.0) <= BOUND


def test_overflow_gives_inf():
    x = np.array([128.0, 128.5, 300.0, 1e30, np.inf], np.float32)
    assert np.all(np.isposinf(emulate(x)))


def test_planted_sign_error_is_caught():
    x = grid()[::50]
    err = rel_err(emulate(x, flip=True), x)
    assert np.isnan(err).any() or np.nanmax(err) > 100 * BOUND

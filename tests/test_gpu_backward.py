"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle.

The GPU path runs as a user would: the library's forward gives O and the
log-sum-exp, the backward takes them with dO.  The oracle computes the
gradients from Q, K, V, dO alone (chain rule through the definition).

Gate, per gradient tensor G: max |G - G_ref| <= GRAD_TOL * max |G_ref|.  The
kernels round P and dS to the 16-bit input type for the matrix cores
(relative error 2^-9 for bf16), build D from the 16-bit O, and round the
result to 16 bits; each contributes errors of order 2^-9 relative to the
largest terms of the sums, a few times 2^-9 ~ 2e-3 in all.  GRAD_TOL = 2e-2
leaves a factor of about five; a wrong mask, index or missing term is off by
O(1).  Every output element is checked to have been written (outputs start
as NaN)."""
import math

import numpy as np
import pytest

import fa_inputs as G
from oracle import backward as BW

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2


@pytest.fixture(scope="module")
def F():
    import torch
    import flashattention_forward_amd as F
    assert torch.cuda.is_available()
    F.lib()
    return F


def _run(F, q, k, v, do, w, causal):
    """forward then backward on the GPU; returns (dq, dk, dv) as fp64 numpy."""
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    tq, tk, tv, tdo = (to_dev(x, w.dtype) for x in (q, k, v, do))
    print(f"  gpu: {w.name} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} causal={causal}", flush=True)
    out, lse = F.attn_fwd(tq, tk, tv, causal=causal, scale=w.scale)
    dq, dk, dv = nan_like(tq), nan_like(tk), nan_like(tv)
    F.attn_bwd(tq, tk, tv, out, tdo, lse, causal=causal, scale=w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return from_dev(dq), from_dev(dk), from_dev(dv)


def _check(got, ref, tol=GRAD_TOL):
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), f"unwritten or non-finite {name}"
        e = float(np.max(np.abs(g - r)))
        m = float(np.max(np.abs(r)))
        errs.append((name, e, m))
        assert e <= tol * m, (name, e, m)
    print("  " + "  ".join(f"max|d{n}|={e:.3e} (max|ref| {m:.3e}, ratio {e / m:.2e})" for n, e, m in errs), flush=True)
    return errs


def _inputs(w, seed=0, heads=None):
    q, k, v = G.draw_qkv(w, seed, heads)
    do = G.draw_tensor(w, "do", seed, heads)
    return q, k, v, do


SMALL = [  # (B, H, Nq, Nk): several tiles of 32 and 128 rows, ragged tails on both sides
    (2, 3, 300, 300), (1, 2, 77, 333), (1, 1, 129, 129), (2, 1, 2, 700), (1, 2, 256, 64), (1, 1, 383, 1000),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_backward_small(F, dtype, d, causal, shape):
    B, H, Nq, Nk = shape
    if causal and Nq > Nk:
        pytest.skip("causal needs Nq <= Nk (rejected before launch, see test_abi)")
    w = G.Workload(f"bwd_{dtype}_{d}", 40 + d + (dtype == "fp16"), B, H, Nq, Nk, d, dtype, 1.0, causal,
                   1 / math.sqrt(d))
    q, k, v, do = _inputs(w)
    f = lambda x: G.to_f64(x, dtype)
    ref = BW.attention_backward(f(q), f(k), f(v), f(do), w.scale, causal)
    _check(_run(F, q, k, v, do, w, causal), ref)


def test_backward_single_key(F):
    """Nk = 1: P is 1 for every query, so dS = 0 (dQ = dK = 0) and dV is the
    sum of the dO rows (closed form).  On the GPU dS is the difference of
    dP = dO . v and D = dO . O with O = v, two fp32 sums of 64 products taken
    in different orders: a few fp32 ulps of |dO| |v| sqrt(64) ~ 10, so dQ and
    dK are bounded by 1e-4 instead of being exactly zero."""
    w = G.Workload("bwd_one_key", 60, 1, 2, 70, 1, 64, "bf16", 1.0, False, 0.125)
    q, k, v, do = _inputs(w)
    dq, dk, dv = _run(F, q, k, v, do, w, False)
    assert np.max(np.abs(dq)) <= 1e-4 and np.max(np.abs(dk)) <= 1e-4
    ref = G.to_f64(do, "bf16").sum(axis=2, keepdims=True)
    assert np.max(np.abs(dv - ref)) <= GRAD_TOL * np.max(np.abs(ref))


def test_backward_is_deterministic(F):
    """No atomics: two runs give the same bits."""
    w = G.Workload("bwd_det", 61, 1, 4, 500, 500, 128, "bf16", 1.0, True, 128 ** -0.5)
    q, k, v, do = _inputs(w)
    a = _run(F, q, k, v, do, w, True)
    b = _run(F, q, k, v, do, w, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_size_sampled(F, causal):
    """B=4 H=32 N=4096 d=128 bf16 (the bench's configuration), all heads on
    the GPU in one call; three heads checked element by element against the
    oracle."""
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    w = G.shrink(G.WORKLOADS["prefill_4k"], causal=causal)
    q, k, v, do = _inputs(w)
    tq, tk, tv, tdo = (to_dev(x, w.dtype) for x in (q, k, v, do))
    print(f"  gpu: full size B={w.B} H={w.H} N={w.Nq} d={w.d} causal={causal}", flush=True)
    out, lse = F.attn_fwd(tq, tk, tv, causal=causal, scale=w.scale)
    dq, dk, dv = nan_like(tq), nan_like(tk), nan_like(tv)
    F.attn_bwd(tq, tk, tv, out, tdo, lse, causal=causal, scale=w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all()), "unwritten or non-finite gradient"
    f = lambda x: G.to_f64(x, w.dtype)
    for (b, h) in [(0, 0), (1, 17), (3, 31)]:
        ref = BW.attention_backward_head(f(q[b, h]), f(k[b, h]), f(v[b, h]), f(do[b, h]), w.scale, causal)
        got = tuple(from_dev(t[b, h]) for t in (dq, dk, dv))
        print(f"  head ({b}, {h})", flush=True)
        _check(got, ref)

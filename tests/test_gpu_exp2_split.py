"""GPU checks of the software-exp2 split (attn_fwd_exp2_split): the prefill
with 2 or 4 of every 8 softmax exponentials on the library's polynomial exp2
instead of v_exp_f32.

* The polynomial, evaluated on the GPU by the routine the kernel calls, stays
  within its relative error bound of the exact 2^x; arguments below -125
  give 0.
* The split forward meets the same gates against the fp64 oracle as the
  default forward: max |O - O_ref| <= 2e-2, max |LSE - LSE_ref| <= 1e-3.
  Small shapes cover both dtypes, both masks, ragged tails and Nq != Nk; the
  prefill workload (B=4 H=32 N=4096) is compared on sampled rows.
* A share of 0 is attn_fwd's own kernel, bit for bit."""
import numpy as np
import pytest

import fa_inputs as G
from oracle import attention as A
from tests.test_exp2_poly import BOUND, grid, rel_err
from tests.test_gpu_prefill import _check, _sampled_heads, _sampled_rows, _whole, LSE_TOL, O_TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    import torch
    import flashattention_forward_amd as F
    assert torch.cuda.is_available()
    F.lib()
    return F


def test_exp2_poly_within_bound(F):
    import torch
    x = grid()
    print(f"  gpu: debug_exp2_poly n={x.size}", flush=True)
    y = F.debug_exp2_poly(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.all(np.isfinite(y)) and np.all(y > 0)
    assert rel_err(y, x).max() <= BOUND
    z = np.array([-125.5, -126.0, -300.0, -np.inf], np.float32)
    assert np.all(F.debug_exp2_poly(torch.from_numpy(z).cuda()).cpu().numpy() == 0.0)
    big = np.array([128.0, 200.0, np.inf], np.float32)
    assert np.all(np.isposinf(F.debug_exp2_poly(torch.from_numpy(big).cuda()).cpu().numpy()))


def _run_split(F, w, causal, poly, seed=0):
    import torch
    from tests.gpu_util import nan_like, to_dev
    q, k, v = G.draw_qkv(w, seed, threads=16)
    tq, tk, tv = (to_dev(x, w.dtype) for x in (q, k, v))
    out = nan_like(tq)
    lse = torch.full((w.B, w.H, w.Nq), float("nan"), device="cuda")
    print(f"  gpu: exp2 split {poly}/8 {w.name} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} {w.dtype} causal={causal}",
          flush=True)
    F.attn_fwd_exp2_split(tq, tk, tv, poly, causal=causal, scale=w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return (q, k, v), out, lse


@pytest.mark.parametrize("poly", [2, 4])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 300, 300), (2, 1, 200, 520), (1, 1, 64, 64)])
def test_exp2_split_small(F, poly, dtype, causal, shape):
    B, H, Nq, Nk = shape
    w = G.Workload("exp2_split_small", 31, B, H, Nq, Nk, 128, dtype, 1.0, causal, 128 ** -0.5)
    _, _, _, O, L = _whole(w, causal, seed=0)
    _, out, lse = _run_split(F, w, causal, poly, seed=0)
    _check(out, lse, O, L)


def test_exp2_split_full_size_sampled(F):
    from tests.gpu_util import from_dev
    w = G.WORKLOADS["prefill_4k"]
    (q, k, v), out, lse = _run_split(F, w, False, 4)
    o_all, l_all = from_dev(out), from_dev(lse)
    assert np.isfinite(o_all).all() and np.isfinite(l_all).all()
    worst_o = worst_l = 0.0
    for (b, h) in _sampled_heads(w, 4):
        rows = _sampled_rows(w.Nq, 32, seed=b * 1000 + h)
        f = lambda x: G.to_f64(x[b, h], w.dtype)
        O, L = A.attention_rows(f(q), f(k), f(v), rows, w.scale, False)
        worst_o = max(worst_o, np.abs(o_all[b, h, rows] - O).max())
        worst_l = max(worst_l, np.abs(l_all[b, h, rows] - L).max())
    print(f"  sampled max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}", flush=True)
    assert worst_o <= O_TOL and worst_l <= LSE_TOL


def test_share_zero_is_the_default_kernel(F):
    import torch
    from tests.gpu_util import to_dev
    w = G.Workload("exp2_split_zero", 32, 1, 3, 700, 700, 128, "bf16", 1.0, True, 128 ** -0.5)
    tq, tk, tv = (to_dev(x, w.dtype) for x in G.draw_qkv(w, 0))
    print("  gpu: share 0 against attn_fwd", flush=True)
    a = F.attn_fwd_exp2_split(tq, tk, tv, 0, causal=True, scale=w.scale)
    b = F.attn_fwd(tq, tk, tv, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])

"""attn_fwd_decode_static, the decode entry point that allocates nothing
(its split partials live in the library's static device scratch), against
attn_fwd_decode with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller problem, so the second reuses
the scratch the first left behind; both must equal the workspace entry
point's result bit for bit (same kernels, same split count) and hold the
dense forward's gates against the fp64 oracle.  (A problem whose partials
exceed the scratch is refused before anything is launched: tests/test_abi.py
checks that on the CPU.)"""
import ctypes
import math

import numpy as np
import pytest

import fa_inputs as G
from oracle import attention as A

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 2e-2, 1e-3
SCRATCH_BYTES = 8 << 20


@pytest.fixture(scope="module")
def F():
    import torch
    import flashattention_forward_amd as F
    assert torch.cuda.is_available()
    F.lib()
    return F


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _run_pair(F, B, H, Nk, d, dtype, splits, seed):
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    from flashattention_forward_amd import binding as Bd
    w = G.Workload(f"decode_static_{B}_{H}_{Nk}", seed, B, H, 1, Nk, d, dtype, 1.0, False, 1 / math.sqrt(d))
    q, k, v = G.draw_qkv(w)
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    code = Bd.ATTN_BF16 if dtype == "bf16" else Bd.ATTN_FP16
    L = F.lib()
    print(f"  gpu: decode static B={B} H={H} Nk={Nk} d={d} {dtype} splits={splits}", flush=True)
    # the entry point under test: no workspace argument
    out_s, lse_s = nan_like(tq), torch.full((B, H, 1), float("nan"), device="cuda")
    rc = L.attn_fwd_decode_static(_p(tq), _p(tk), _p(tv), _p(out_s), _p(lse_s), B, H, Nk, d, w.scale, code, splits,
                                  _stream())
    assert rc == Bd.ATTN_OK, Bd.status_str(rc)
    # the existing entry point with a caller workspace
    wsb = int(L.attn_decode_workspace_bytes(B, H, d, splits))
    assert wsb <= SCRATCH_BYTES
    ws = torch.empty(wsb, device="cuda", dtype=torch.uint8)
    out_w, lse_w = nan_like(tq), torch.full((B, H, 1), float("nan"), device="cuda")
    rc = L.attn_fwd_decode(_p(tq), _p(tk), _p(tv), _p(out_w), _p(lse_w), B, H, Nk, d, w.scale, code, splits, _p(ws),
                           wsb, _stream())
    assert rc == Bd.ATTN_OK, Bd.status_str(rc)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w) and torch.equal(lse_s, lse_w), "static scratch differs from the workspace call"
    O, Lr = A.attention(*(G.to_f64(x, dtype) for x in (q, k, v)), w.scale, False)
    o, l = from_dev(out_s), from_dev(lse_s)
    eo, el = float(np.max(np.abs(o - O))), float(np.max(np.abs(l - Lr)))
    print(f"  max|dO|={eo:.3e}  max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_static_decode_two_calls(F, dtype, d):
    # the larger call fills most of the scratch; the smaller one follows it
    B, H, Nk = 16, 32, 2048
    splits = 16
    assert B * H * splits * (d + 1) * 4 <= SCRATCH_BYTES
    _run_pair(F, B, H, Nk, d, dtype, splits, seed=31 + d)
    _run_pair(F, 3, 5, 300, d, dtype, 3, seed=37 + d)

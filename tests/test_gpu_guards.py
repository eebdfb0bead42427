"""Guard regions around every output the library writes: each output (O,
LSE, the decode workspace, the backward's gradients and workspace, the
quantised forwards' outputs, the quantisers' codes and scales) is placed
inside a larger buffer with 4 KiB of canary bytes on each side, and after the
call every canary byte must be unchanged, so no kernel writes outside its
outputs.  Shapes are small and ragged (tails past every tile size), both
masks, both head sizes.  Outputs start as NaN and must come back finite
(every element written)."""
import math

import numpy as np
import pytest

import fa_inputs as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    import torch
    import flashattention_forward_amd as F
    assert torch.cuda.is_available()
    F.lib()
    return F


def _qkv(dtype, B, H, Hkv, Nq, Nk, d, seed):
    from tests.gpu_util import to_dev
    wq = G.Workload(f"guard_{seed}", 300 + seed, B, H, Nq, Nk, d, dtype, 1.0, False, 1 / math.sqrt(d))
    wk = G.shrink(wq, H=Hkv)
    return (to_dev(G.draw_tensor(wq, "q"), dtype), to_dev(G.draw_tensor(wk, "k"), dtype),
            to_dev(G.draw_tensor(wk, "v"), dtype))


def _finite(t):
    import torch
    return bool(torch.isfinite(t.float()).all())


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 300, 300), (2, 4, 2, 77, 333), (1, 3, 3, 1, 515)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_outputs_guarded(F, dtype, d, causal, shape):
    import torch
    from flashattention_forward_amd import binding as Bd
    from tests.gpu_util import Guarded
    B, H, Hkv, Nq, Nk = shape
    q, k, v = _qkv(dtype, B, H, Hkv, Nq, Nk, d, seed=d + 2 * causal + (dtype == "fp16"))
    out = Guarded(q.shape, q.dtype)
    lse = Guarded((B, H, Nq), torch.float32)
    wsb = Bd.workspace_bytes(B, H, Nq, Nk, d, Bd.ATTN_BF16 if dtype == "bf16" else Bd.ATTN_FP16, Hkv)
    ws = Guarded((max(wsb, 16),), torch.uint8, fill=0xEE) if wsb else None
    print(f"  gpu: guarded attn_fwd {shape} d={d} {dtype} causal={causal}", flush=True)
    F.attn_fwd(q, k, v, causal=causal, out=out.t, lse=lse.t, workspace=ws.t if ws else None)
    torch.cuda.synchronize()
    assert out.intact() and lse.intact() and (ws is None or ws.intact())
    assert _finite(out.t) and _finite(lse.t)


def test_decode_and_static_decode_guarded(F):
    import ctypes
    import torch
    from flashattention_forward_amd import binding as Bd
    from tests.gpu_util import Guarded
    B, H, Nk, d = 3, 5, 700, 128
    q, k, v = _qkv("bf16", B, H, H, 1, Nk, d, seed=40)
    for splits in (1, 3, 7):
        out, lse = Guarded(q.shape, q.dtype), Guarded((B, H, 1), torch.float32)
        wsb = int(F.lib().attn_decode_workspace_bytes(B, H, d, splits))
        ws = Guarded((wsb,), torch.uint8, fill=0xEE)
        print(f"  gpu: guarded decode splits={splits}", flush=True)
        F.attn_fwd_decode(q, k, v, splits, out=out.t, lse=lse.t, workspace=ws.t)
        torch.cuda.synchronize()
        assert out.intact() and lse.intact() and ws.intact() and _finite(out.t) and _finite(lse.t)
    out, lse = Guarded(q.shape, q.dtype), Guarded((B, H, 1), torch.float32)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = F.lib().attn_fwd_decode_static(p(q), p(k), p(v), p(out.t), p(lse.t), B, H, Nk, d, 1 / math.sqrt(d),
                                        Bd.ATTN_BF16, 4, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0 and out.intact() and lse.intact() and _finite(out.t)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_outputs_guarded(F, causal):
    import torch
    from tests.gpu_util import Guarded
    lq, lk = [5, 0, 130, 77], [9, 20, 200, 77]
    if causal:
        lk = [max(a, b) for a, b in zip(lq, lk)]
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32, device="cuda")
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32, device="cuda")
    q, k, v = _qkv("bf16", 1, 4, 2, sum(lq), sum(lk), 64, seed=50 + causal)
    q, k, v = q[0], k[0], v[0]
    out, lse = Guarded(q.shape, q.dtype), Guarded((4, sum(lq)), torch.float32)
    print(f"  gpu: guarded varlen causal={causal}", flush=True)
    F.attn_fwd_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=causal, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    assert out.intact() and lse.intact() and _finite(out.t)
    dq, dk, dv = Guarded(q.shape, q.dtype), Guarded(k.shape, k.dtype), Guarded(v.shape, v.dtype)
    ws = Guarded((4 * sum(lq) * 8,), torch.uint8, fill=0xEE)
    F.attn_bwd_varlen(q, k, v, out.t, out.t.clone(), lse.t, cq, ck, max(lq), max(lk), causal=causal, dq=dq.t,
                      dk=dk.t, dv=dv.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert dq.intact() and dk.intact() and dv.intact() and ws.intact()
    assert _finite(dq.t) and _finite(dk.t) and _finite(dv.t)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_outputs_guarded(F, d, causal):
    import torch
    from tests.gpu_util import Guarded
    B, H, Hkv, Nq, Nk = 1, 4, 2, 200, 333
    q, k, v = _qkv("bf16", B, H, Hkv, Nq, Nk, d, seed=60 + d + causal)
    out, lse = F.attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = Guarded(q.shape, q.dtype), Guarded(k.shape, k.dtype), Guarded(v.shape, v.dtype)
    wsb = int(F.lib().attn_bwd_workspace_bytes(B, H, Nq, Nk, d, 0))
    ws = Guarded((wsb,), torch.uint8, fill=0xEE)
    print(f"  gpu: guarded backward d={d} causal={causal}", flush=True)
    F.attn_bwd(q, k, v, out, out.clone(), lse, causal=causal, dq=dq.t, dk=dk.t, dv=dv.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert dq.intact() and dk.intact() and dv.intact() and ws.intact()
    assert _finite(dq.t) and _finite(dk.t) and _finite(dv.t)


@pytest.mark.parametrize("causal", [False, True])
def test_quantised_outputs_guarded(F, causal):
    import torch
    from tests.gpu_util import Guarded
    B, H, Nq, Nk, d = 1, 2, 130, 333, 128
    q, k, v = _qkv("bf16", B, H, H, Nq, Nk, d, seed=70 + causal)
    # quantisers: codes and scales guarded
    q8, sq = Guarded(q.shape, torch.int8, fill=0), Guarded((B, H, Nq), torch.float32)
    import ctypes
    from flashattention_forward_amd import binding as Bd
    rc = F.lib().attn_quantize_rows_i8(*(ctypes.c_void_p(t.data_ptr()) for t in (q, q8.t, sq.t)),
                                       q.numel() // d, d, Bd._stream())
    torch.cuda.synchronize()
    assert rc == 0 and q8.intact() and sq.intact() and _finite(sq.t)
    k8, sk = F.quantize_rows_i8(k)
    v8, sv = F.quantize_tensor_e4m3(v)
    vi8, svi = F.quantize_tensor_i8(v)
    signs = torch.tensor(np.where(np.random.default_rng(3).random(d) < 0.5, -1.0, 1.0), dtype=torch.float32,
                         device="cuda")
    qf8, sqf = F.rotate_quantize_e4m3(q, signs)
    kf8, skf = F.rotate_quantize_e4m3(k, signs)
    runs = [("q8", F.attn_fwd_q8, (q8.t, k8, v8, sq.t, sk, sv)),
            ("i8", F.attn_fwd_i8, (q8.t, k8, vi8, sq.t, sk, svi)),
            ("fp8", F.attn_fwd_fp8, (qf8, kf8, v8, sqf, skf, sv)),
            ("fp4p", F.attn_fwd_fp4p, (qf8, kf8, v8, sqf, skf, sv))]
    for name, fn, args in runs:
        out, lse = Guarded((B, H, Nq, d), torch.bfloat16), Guarded((B, H, Nq), torch.float32)
        print(f"  gpu: guarded {name} causal={causal}", flush=True)
        fn(*args, causal=causal, out=out.t, lse=lse.t)
        torch.cuda.synchronize()
        assert out.intact() and lse.intact() and _finite(out.t) and _finite(lse.t), name

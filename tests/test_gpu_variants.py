"""GPU parity of grouped-query (GQA/MQA) and packed variable-length (varlen)
attention against the fp64 oracle (oracle.variants), through the C ABI.
Gates as for the dense forward: max |O - O_ref| <= 2e-2, max |LSE - LSE_ref|
<= 1e-3; rows that see no key must be exactly O = 0, LSE = -inf; every
output element is checked to have been written (outputs start as NaN)."""
import math

import numpy as np
import pytest

import fa_inputs as G
from oracle import variants as V

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 2e-2, 1e-3


@pytest.fixture(scope="module")
def F():
    import torch
    import flashattention_forward_amd as F
    assert torch.cuda.is_available()
    F.lib()
    return F


def _check(o, l, O, L):
    assert np.isfinite(o).all(), "unwritten or non-finite outputs"
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(l), fin), "LSE finiteness differs from the oracle"
    assert np.all(l[~fin] == -np.inf) and np.all(o[~fin] == 0.0), "rows with no key must be O = 0, LSE = -inf"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(l[fin] - L[fin]))) if fin.any() else 0.0
    print(f"  max|dO|={eo:.3e}  max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


GQA = [  # (B, H, Hkv, Nq, Nk)
    (2, 8, 2, 300, 300), (1, 4, 1, 77, 333), (1, 6, 3, 129, 129), (2, 4, 2, 2, 700), (1, 8, 1, 600, 600),
    # Nq = 1: the split-KV decode path, whose workgroups serve 8, 4, 2 or 1 query
    # heads of a group together (group 4, 8, 2, 3 and MQA with 16 heads)
    (3, 8, 2, 1, 1000), (2, 16, 2, 1, 777), (2, 6, 3, 1, 300), (1, 6, 2, 1, 4099), (2, 16, 1, 1, 513),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", GQA, ids=lambda s: "x".join(map(str, s)))
def test_gqa(F, dtype, d, causal, shape):
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    B, H, Hkv, Nq, Nk = shape
    if causal and Nq > Nk:
        pytest.skip("causal needs Nq <= Nk")
    wq = G.Workload(f"gqa_{dtype}_{d}", 70 + d + (dtype == "fp16"), B, H, Nq, Nk, d, dtype, 1.0, causal,
                    1 / math.sqrt(d))
    wk = G.shrink(wq, H=Hkv)
    q = G.draw_tensor(wq, "q")
    k, v = G.draw_tensor(wk, "k"), G.draw_tensor(wk, "v")
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    out = nan_like(tq)
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    print(f"  gpu: GQA B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}", flush=True)
    F.attn_fwd(tq, tk, tv, causal=causal, scale=wq.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    f = lambda x: G.to_f64(x, dtype)
    O, L = V.attention_gqa(f(q), f(k), f(v), wq.scale, causal)
    _check(from_dev(out), from_dev(lse), O, L)


VARLEN = [  # (query lengths, key lengths, H, Hkv)
    ([300, 17, 256, 1, 700], [300, 40, 256, 9, 700], 4, 2),
    ([5, 0, 513, 64], [5, 33, 513, 64], 2, 1),
    ([100, 50, 3], [0, 20, 3], 2, 2),            # an empty key range; causal: more queries than keys
    ([1000], [1200], 3, 3),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen(F, dtype, d, causal, case):
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    lq, lk, H, Hkv = VARLEN[case]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    tq_, tk_ = int(cq[-1]), int(ck[-1])
    wq = G.Workload(f"varlen_{dtype}_{d}", 80 + d + (dtype == "fp16") + 2 * case, 1, H, tq_, tk_, d, dtype, 1.0,
                    causal, 1 / math.sqrt(d))
    wk = G.shrink(wq, H=Hkv)
    q = G.draw_tensor(wq, "q")[0]
    k, v = G.draw_tensor(wk, "k")[0], G.draw_tensor(wk, "v")[0]
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    out = nan_like(tq)
    lse = torch.full((H, tq_), float("nan"), device="cuda")
    print(f"  gpu: varlen lq={lq} lk={lk} H={H} Hkv={Hkv} d={d} {dtype} causal={causal}", flush=True)
    F.attn_fwd_varlen(tq, tk, tv, torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), max(lq), max(lk),
                      causal=causal, scale=wq.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    f = lambda x: G.to_f64(x, dtype)
    O, L = V.attention_varlen(f(q), f(k), f(v), cq, ck, wq.scale, causal)
    _check(from_dev(out), from_dev(lse), O, L)


def test_gqa_full_size_sampled(F):
    """B=4 H=32 Hkv=8 N=4096 d=128 bf16 causal (the GQA bench configuration):
    whole launch on the GPU, sampled rows of sampled heads against the oracle."""
    import torch
    from oracle import attention as A
    from tests.gpu_util import from_dev, to_dev
    w = G.WORKLOADS["gqa_4k_causal"]
    q = G.draw_tensor(w, "q", threads=16)
    wk = G.shrink(w, H=8)
    k, v = G.draw_tensor(wk, "k", threads=16), G.draw_tensor(wk, "v", threads=16)
    out, lse = F.attn_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    f = lambda x: G.to_f64(x, "bf16")
    for (b, h) in [(0, 0), (1, 13), (3, 31)]:
        g = V.kv_head(h, 32, 8)
        O, L = A.attention_rows(f(q[b, h]), f(k[b, g]), f(v[b, g]), rows, w.scale, True)
        eo = np.max(np.abs(from_dev(out[b, h])[rows] - O))
        el = np.max(np.abs(from_dev(lse[b, h])[rows] - L))
        print(f"  head ({b},{h}) -> kv {g}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        assert eo <= O_TOL and el <= LSE_TOL


# ---------------------------------------------------------------- backward
# Gate as for the dense backward: max |G - G_ref| <= GRAD_TOL * max |G_ref| per
# gradient tensor (P and dS are rounded to 16 bits for the matrix cores).
GRAD_TOL = 2e-2


def _check_grads(got, ref):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), f"unwritten or non-finite {name}"
        e, m = float(np.max(np.abs(g - r))), float(np.max(np.abs(r)))
        print(f"  {name}: max err {e:.3e} (max |ref| {m:.3e})", flush=True)
        assert e <= GRAD_TOL * m, (name, e, m)


GQA_BWD = [(2, 8, 2, 300, 300), (1, 4, 1, 77, 333), (1, 6, 3, 129, 129), (1, 8, 4, 256, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", GQA_BWD, ids=lambda s: "x".join(map(str, s)))
def test_gqa_backward(F, dtype, d, causal, shape):
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    B, H, Hkv, Nq, Nk = shape
    if causal and Nq > Nk:
        pytest.skip("causal needs Nq <= Nk")
    wq = G.Workload(f"gqa_bwd_{dtype}_{d}", 90 + d + (dtype == "fp16"), B, H, Nq, Nk, d, dtype, 1.0, causal,
                    1 / math.sqrt(d))
    wk = G.shrink(wq, H=Hkv)
    q, do = G.draw_tensor(wq, "q"), G.draw_tensor(wq, "do")
    k, v = G.draw_tensor(wk, "k"), G.draw_tensor(wk, "v")
    tq, tk, tv, tdo = (to_dev(x, dtype) for x in (q, k, v, do))
    print(f"  gpu: GQA bwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}", flush=True)
    out, lse = F.attn_fwd(tq, tk, tv, causal=causal, scale=wq.scale)
    dq, dk, dv = nan_like(tq), nan_like(tk), nan_like(tv)
    F.attn_bwd(tq, tk, tv, out, tdo, lse, causal=causal, scale=wq.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    f = lambda x: G.to_f64(x, dtype)
    ref = V.attention_backward_gqa(f(q), f(k), f(v), f(do), wq.scale, causal)
    _check_grads(tuple(from_dev(t) for t in (dq, dk, dv)), ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen_backward(F, dtype, d, causal, case):
    import torch
    from tests.gpu_util import from_dev, nan_like, to_dev
    lq, lk, H, Hkv = VARLEN[case]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    tq_, tk_ = int(cq[-1]), int(ck[-1])
    wq = G.Workload(f"varlen_bwd_{dtype}_{d}", 100 + d + (dtype == "fp16") + 2 * case, 1, H, tq_, tk_, d, dtype,
                    1.0, causal, 1 / math.sqrt(d))
    wk = G.shrink(wq, H=Hkv)
    q, do = G.draw_tensor(wq, "q")[0], G.draw_tensor(wq, "do")[0]
    k, v = G.draw_tensor(wk, "k")[0], G.draw_tensor(wk, "v")[0]
    tq, tk, tv, tdo = (to_dev(x, dtype) for x in (q, k, v, do))
    cu_q, cu_k = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    print(f"  gpu: varlen bwd lq={lq} lk={lk} H={H} Hkv={Hkv} d={d} {dtype} causal={causal}", flush=True)
    out, lse = F.attn_fwd_varlen(tq, tk, tv, cu_q, cu_k, max(lq), max(lk), causal=causal, scale=wq.scale)
    dq, dk, dv = nan_like(tq), nan_like(tk), nan_like(tv)
    F.attn_bwd_varlen(tq, tk, tv, out, tdo, lse, cu_q, cu_k, max(lq), max(lk), causal=causal, scale=wq.scale,
                      dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    f = lambda x: G.to_f64(x, dtype)
    ref = V.attention_backward_varlen(f(q), f(k), f(v), f(do), cq, ck, wq.scale, causal)
    got = tuple(from_dev(t) for t in (dq, dk, dv))
    # rows that see no key: exactly zero gradient
    _, L = V.attention_varlen(f(q), f(k), f(v), cq, ck, wq.scale, causal)
    assert np.all(got[0][~np.isfinite(L)] == 0.0)
    _check_grads(got, ref)


def test_varlen_backward_without_queries(F):
    """A packed batch whose sequences hold keys but no query at all
    (total_q = 0, total_k > 0): the backward returns 0 and writes dK = dV = 0.
    The query-side tensors are empty, so the call goes through the C ABI with
    small stand-in buffers for them (the library reads no query row)."""
    import ctypes
    import torch
    from flashattention_forward_amd import binding as Bd
    H, Hkv, d = 2, 1, 64
    ck = torch.tensor([0, 5, 135], dtype=torch.int32, device="cuda")
    cq = torch.zeros(3, dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(11)
    k = torch.randn(Hkv, 135, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(Hkv, 135, d, generator=g).to(torch.bfloat16).cuda()
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    stand_in = torch.zeros(64, device="cuda", dtype=torch.bfloat16)
    lse_in = torch.zeros(16, device="cuda", dtype=torch.float32)
    ws = torch.zeros(64, device="cuda", dtype=torch.uint8)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    print("  gpu: varlen bwd, 2 sequences, keys (5, 130), no queries", flush=True)
    rc = Bd.lib().attn_bwd_varlen(p(stand_in), p(k), p(v), p(stand_in), p(stand_in), p(lse_in), p(stand_in), p(dk),
                                  p(dv), p(cq), p(ck), 2, 0, 130, 0, 135, H, Hkv, d, 0.125, 0, Bd.ATTN_BF16, p(ws),
                                  64, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == Bd.ATTN_OK, Bd.status_str(rc)
    assert bool((dk == 0).all()) and bool((dv == 0).all())

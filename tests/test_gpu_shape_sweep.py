"""GPU parity of attn_fwd over a seeded sweep of shapes, against the fp64
oracle: batch and head counts (grouped-query heads included) up to grids that
take the persistent and paired launches, lengths with ragged last blocks,
Nq <= Nk for causal, both head sizes and both dtypes.  Every output element
is compared (O within 2e-2, LSE within 1e-3, as for the other prefill tests)
and must have been written (outputs start as NaN)."""
import numpy as np
import pytest

import fa_inputs as G
from oracle import variants as V

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 2e-2, 1e-3
MAX_WORK = 3.0e9     # B*H*Nq*Nk*d per case, so the fp64 oracle stays at seconds


def _cases(n=24, seed=20261204):
    """Seeded cases; every fourth is a dense non-causal grid with more query
    blocks than CUs (the persistent launch), every fourth (offset by two) a
    causal grid of 1024 (batch, head) pairs (the paired persistent launch)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = len(out) % 4
        if kind == 1:
            B, H, d, causal = 2, int(rng.choice([130, 160])), 128, False
            Nk = int(rng.integers(2, 140))
            Nq = int(rng.integers(257, 521))
        elif kind == 3:
            B, H, d, causal = 4, 256, 128, True
            Nk = int(rng.integers(2, 151))
            Nq = int(rng.integers(2, Nk + 1))
        else:
            B = int(rng.choice([1, 2, 4]))
            H = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32]))
            d = int(rng.choice([64, 128]))
            causal = bool(rng.integers(0, 2))
            Nk = int(rng.integers(2, 1300))
            Nq = int(rng.integers(2, Nk + 1)) if causal else int(rng.integers(2, 1300))
        divs = [g for g in range(1, H + 1) if H % g == 0 and g <= 32]
        Hkv = H // int(rng.choice(divs))
        dtype = str(rng.choice(["bf16", "fp16"]))
        if B * H * Nq * Nk * d > MAX_WORK:
            continue
        out.append((B, H, Hkv, Nq, Nk, d, dtype, causal))
    return out


@pytest.fixture(scope="module")
def F():
    import torch
    import flashattention_forward_amd as F
    assert torch.cuda.is_available()
    F.lib()
    return F


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{}H{}kv{}q{}k{}d{}{}{}".format(*c[:7], "c" if c[7] else ""))
def test_shape_sweep(F, case):
    import torch
    from tests.gpu_util import errors, from_dev, nan_like, to_dev
    B, H, Hkv, Nq, Nk, d, dtype, causal = case
    w = G.Workload("shape_sweep", 62, B, H, Nq, Nk, d, dtype, 1.0, causal, d ** -0.5)
    q = G.draw_tensor(w, "q", threads=16)
    wk = G.shrink(w, H=Hkv)
    k, v = (G.draw_tensor(wk, t, threads=16) for t in ("k", "v"))
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    out = nan_like(tq)
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    print(f"  gpu: shape sweep B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}", flush=True)
    F.attn_fwd(tq, tk, tv, causal=causal, scale=w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    f = lambda x: G.to_f64(x, dtype)
    O, L = V.attention_gqa(f(q), f(k), f(v), w.scale, causal)
    o, l = from_dev(out), from_dev(lse)
    assert np.isfinite(o).all() and np.isfinite(l).all(), "unwritten or non-finite outputs"
    eo, _ = errors(o, O)
    el, _ = errors(l, L)
    print(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL

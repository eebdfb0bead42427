"""The seeded input generator (no GPU)."""
import numpy as np
import torch

import fa_inputs as G


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(50000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(50000) * 1e30).astype(np.float32)])
    # exact ties: low 16 bits 0x8000 with odd and even kept parts
    u = rng.integers(0, 2 ** 31, 4000, dtype=np.uint32) & np.uint32(0x7F7F0000) | np.uint32(0x8000)
    x = np.concatenate([x, u.view(np.float32), -u.view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(G.round_to_bf16_bits(x), ref)


def test_bf16_widening_is_exact_for_all_patterns():
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = G.bf16_bits_to_f32(bits)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()


def test_heads_are_independent_streams():
    w = G.shrink(G.WORKLOADS["prefill_4k"], B=2, H=3, Nq=40, Nk=40)
    q, k, v = G.draw_qkv(w, seed=0)
    sub = G.draw_tensor(w, "k", 0, heads=[(1, 2), (0, 1)])
    assert np.array_equal(sub[0], k[1, 2]) and np.array_equal(sub[1], k[0, 1])
    q2, _, _ = G.draw_qkv(w, seed=0, threads=1)
    assert np.array_equal(q, q2)
    assert not np.array_equal(q[0, 0], k[0, 0])
    q3 = G.draw_tensor(w, "q", seed=1)
    assert not np.array_equal(q, q3)


def test_distribution_and_storage():
    w = G.WORKLOADS["long_23400_causal"]
    x = G.draw_tensor(w, "q", heads=[(0, 0)])
    assert x.dtype == np.float16 and x.shape == (1, 23400, 64)
    f = G.to_f64(x, "fp16")
    assert abs(f.mean()) < 0.01 and abs(f.std() - 0.5) < 0.01
    w = G.WORKLOADS["single_head_256"]
    q, k, v = G.draw_qkv(w)
    assert q.dtype == np.uint16 and q.shape == (1, 1, 256, 64)
    f = G.to_f64(v, "bf16")
    assert abs(f.std() - 1.0) < 0.02
    # fp16 storage rounds once from the fp32 draw
    rng = np.random.default_rng([0, w.wid, 0, 0, 0])
    z = rng.standard_normal((256, 64), dtype=np.float32)
    assert np.array_equal(G.to_f32(q[0, 0], "bf16"),
                          torch.from_numpy(z).to(torch.bfloat16).to(torch.float32).numpy())


def test_workload_flops():
    assert G.WORKLOADS["prefill_4k"].flops() == 4 * 4 * 32 * 4096 * 4096 * 128
    assert G.WORKLOADS["prefill_4k_causal"].flops() == 2 * 4 * 32 * 4096 * 4096 * 128

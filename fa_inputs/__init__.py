"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the GPU path's tests and bench and by the CPU
oracle's tests.  It draws numbers and rounds them to the storage type; it
holds none of the attention arithmetic (no products, no softmax, no
quantisation of the method).

Recipe (every tensor of every workload):
  * one numpy PCG64 stream per (workload id, tensor id, batch, head):
    ``np.random.default_rng([seed, workload_id, tensor_id, b, h])`` with
    tensor ids Q=0, K=1, V=2 and, for the backward pass, the upstream
    gradient dO=3 (shaped like Q), so any single head can be regenerated
    alone;
  * ``standard_normal(dtype=float32)`` of shape [N, d], times sigma in fp32;
  * one round-to-nearest-even to the storage type (bf16 via the bit pattern,
    fp16 via numpy's IEEE conversion) -- no double rounding through fp64.

bf16 tensors are returned as ``uint16`` bit patterns and fp16 tensors as
``float16`` arrays; ``to_f64`` widens either one exactly.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-forward problem: sizes, storage dtype and draw recipe."""
    name: str
    wid: int          # workload id, part of every seed
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str        # "bf16" or "fp16"
    sigma: float      # standard deviation of the normal draw
    causal: bool
    scale: float

    def flops(self) -> float:
        """Algorithmic FLOPs: 2*Nq*Nk*d for QK^T plus the same for PV, per
        head; causal (square) counts exactly half."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2.0 if self.causal else f


# The five workloads of this project (sizes from the problem statement), and
# grouped-query variants of two of them:
WORKLOADS = {
    # single head smoke case: B=1 H=1 N=256 d=64 bf16 N(0,1), non-causal
    "single_head_256": Workload("single_head_256", 0, 1, 1, 256, 256, 64, "bf16", 1.0, False, 1.0 / 8.0),
    # prefill: B=4 H=32 N=4096 d=128 bf16 N(0,1), non-causal and causal
    "prefill_4k": Workload("prefill_4k", 1, 4, 32, 4096, 4096, 128, "bf16", 1.0, False, 128 ** -0.5),
    "prefill_4k_causal": Workload("prefill_4k_causal", 1, 4, 32, 4096, 4096, 128, "bf16", 1.0, True, 128 ** -0.5),
    # one trading day at 1 s resolution: B=1 H=12 N=23400 d=64 fp16 N(0, 0.5^2), causal
    "long_23400_causal": Workload("long_23400_causal", 2, 1, 12, 23400, 23400, 64, "fp16", 0.5, True, 1.0 / 8.0),
    # decode: B=64 H=32, one query against 8192 cached keys, d=128 bf16, split-KV
    "decode_8k": Workload("decode_8k", 3, 64, 32, 1, 8192, 128, "bf16", 1.0, False, 128 ** -0.5),
    # quantised: B=2 H=32 N=8192 d=128, int8 Q/K per token, e4m3 V per tensor
    "quant_8k": Workload("quant_8k", 4, 2, 32, 8192, 8192, 128, "bf16", 1.0, False, 128 ** -0.5),
    # grouped-query variants of the prefill and decode shapes: 32 query heads on
    # 8 K/V heads (K/V tensors are drawn with H = 8 via shrink(w, H=8))
    "gqa_4k_causal": Workload("gqa_4k_causal", 5, 4, 32, 4096, 4096, 128, "bf16", 1.0, True, 128 ** -0.5),
    "gqa_decode_8k": Workload("gqa_decode_8k", 6, 64, 32, 1, 8192, 128, "bf16", 1.0, False, 128 ** -0.5),
}


def round_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even.
    Inputs here are finite draws, so NaN/Inf handling is not needed."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor (bf16 bits or fp16) to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    raise ValueError(dtype)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor (bf16 bits or fp16) to fp32."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    raise ValueError(dtype)


def draw_head(seed: int, wid: int, tensor: str, b: int, h: int, n: int, d: int,
              sigma: float, dtype: str) -> np.ndarray:
    """One head of one tensor, [n, d], in its storage representation."""
    rng = np.random.default_rng([seed, wid, TENSOR_ID[tensor], b, h])
    z = rng.standard_normal((n, d), dtype=np.float32)
    if sigma != 1.0:
        z = z * np.float32(sigma)
    if dtype == "bf16":
        return round_to_bf16_bits(z)
    if dtype == "fp16":
        return z.astype(np.float16)
    raise ValueError(dtype)


def draw_tensor(w: Workload, tensor: str, seed: int = 0, heads=None,
                threads: int = 8) -> np.ndarray:
    """A whole tensor [B, H, N, d] (or the listed (b, h) heads stacked as
    [len(heads), N, d]) in its storage representation."""
    n = w.Nq if tensor in ("q", "do") else w.Nk
    store = np.uint16 if w.dtype == "bf16" else np.float16
    if heads is not None:
        out = np.empty((len(heads), n, w.d), dtype=store)
        for i, (b, h) in enumerate(heads):
            out[i] = draw_head(seed, w.wid, tensor, b, h, n, w.d, w.sigma, w.dtype)
        return out
    out = np.empty((w.B, w.H, n, w.d), dtype=store)

    def fill(bh):
        b, h = divmod(bh, w.H)
        out[b, h] = draw_head(seed, w.wid, tensor, b, h, n, w.d, w.sigma, w.dtype)

    if w.B * w.H == 1 or threads <= 1:
        for bh in range(w.B * w.H):
            fill(bh)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(w.B * w.H)))
    return out


def draw_qkv(w: Workload, seed: int = 0, heads=None, threads: int = 8):
    """(q, k, v) for a workload, see ``draw_tensor``."""
    return tuple(draw_tensor(w, t, seed, heads, threads) for t in ("q", "k", "v"))


def shrink(w: Workload, **kw) -> Workload:
    """A smaller workload with the same distribution and a new name/id mix."""
    return dataclasses.replace(w, **kw)


def to_torch(x: np.ndarray, dtype: str, device: str = "cuda"):
    """A stored tensor (bf16 bits as uint16, or fp16) as a torch tensor of
    that dtype on ``device`` (a bit-for-bit copy)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "fp16":
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    raise ValueError(dtype)


def draw_signs(seed: int, d: int) -> np.ndarray:
    """d random signs (+1.0 / -1.0, float32): the diagonal of the random
    rotation applied to Q and K before FP8 block quantisation."""
    rng = np.random.default_rng([seed, 0x5167])
    return np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def outlier_qkv(seed: int, N: int, d: int, kind: str):
    """One head of Q, K, V [N, d] as bf16 bits, N(0, 1) entries with
    outliers: 'sparse' sets 0.1 % of the entries of each tensor to N(0, 10)
    draws; 'channel' multiplies four fixed channels of Q and K by 10 (the
    same channels for every token); 'none' adds nothing."""
    if kind not in ("sparse", "channel", "none"):
        raise ValueError(kind)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    if kind == "sparse":
        q, k, v = (np.where(rng.random(x.shape) < 1e-3, rng.standard_normal(x.shape) * 10, x) for x in (q, k, v))
    elif kind == "channel":
        ch = rng.choice(d, 4, replace=False)
        q[:, ch] *= 10
        k[:, ch] *= 10
    return tuple(round_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))

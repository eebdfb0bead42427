"""Helpers for the GPU tests: numpy <-> torch device tensors for the stored
input formats, and error summaries."""
import numpy as np
import torch

import fa_inputs as G


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored tensor (bf16 bits as uint16, or fp16) -> GPU tensor."""
    return G.to_torch(x, dtype, "cuda")


def from_dev(t: torch.Tensor) -> np.ndarray:
    """GPU bf16/fp16/fp32 tensor -> fp64 numpy (exact widening)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return G.to_f64(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    if t.dtype == torch.float16:
        return t.numpy().astype(np.float64)
    return t.numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    """(max abs error, max relative error) -- the validation protocol asks
    for the largest relative error; the gates use the absolute one."""
    d = np.abs(got - ref)
    return float(d.max()), float((d / np.maximum(np.abs(ref), 1e-6)).max())


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full_like(t, float("nan"))

"""Thin ctypes binding of libattn_mi355x.so.

Argument marshalling only: torch allocates device memory and supplies the
current HIP stream; every step of the attention computation runs in the
library's kernels.  If the library is missing the import fails loudly --
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_mi355x.so")

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP = 0, -1, -2, -3, -4
ATTN_BF16, ATTN_FP16 = 0, 1

# Every symbol include/attn_mi355x.h declares, with its ctypes signature.
_P, _I, _L, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "attn_fwd_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "attn_fwd_gqa_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_fwd_gqa": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_fwd_decode_splits": (_I, [_I, _I, _I, _I]),
    "attn_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "attn_fwd_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "attn_fwd_decode_static": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_bwd_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "attn_bwd_gqa": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "attn_bwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                             _P, _Z, _P]),
    "attn_quantize_rows_i8": (_I, [_P, _P, _P, _L, _I, _P]),
    "attn_quantize_e4m3_workspace_bytes": (_Z, [_L]),
    "attn_quantize_tensor_e4m3": (_I, [_P, _P, _P, _L, _P, _Z, _P]),
    "attn_fwd_q8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_fwd_i8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_quantize_tensor_i8": (_I, [_P, _P, _P, _L, _P, _Z, _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_rotate_quantize_e4m3": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_fwd_fp4p": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_debug_cvt_e2m1": (_I, [_P, _P, _L, _P]),
    "attn_fwd_exp2_split": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "attn_debug_exp2_poly": (_I, [_P, _P, _L, _P]),
    "attn_debug_qk_i32": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "attn_debug_qk_f8": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "attn_debug_cvt_e4m3": (_I, [_P, _P, _L, _P]),
    "attn_status_str": (ctypes.c_char_p, [_I]),
    "attn_build_info": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m flashattention_forward_amd.build` "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(rc: int) -> str:
    return lib().attn_status_str(rc).decode()


def build_info() -> str:
    return lib().attn_build_info().decode()


def _check(rc: int, what: str):
    if rc != ATTN_OK:
        raise RuntimeError(f"{what}: {status_str(rc)} (code {rc})")


# --------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    cur = _torch().cuda.current_device()
    if t.device.index != cur:
        # the library launches on the current device's stream
        raise ValueError(f"{name} is on {t.device} but the current device is cuda:{cur}")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_FP16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(t, name, shape=None, dtype=None, numel=None):
    """Shape, dtype and size checks of a caller's tensor, before any pointer
    is taken: the kernels read and write through raw pointers sized by the
    other arguments, so a mismatched tensor would be accessed out of bounds."""
    if t is None:
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need_workspace(ws, need: int, name: str = "workspace"):
    if ws is not None and _nbytes(ws) < need:
        raise ValueError(f"{name} holds {_nbytes(ws)} bytes, {need} needed")
    return ws


def _need_offsets(cu_q, cu_k):
    """Packed-batch offsets: int32, one dimension, nseq + 1 >= 2 entries each."""
    torch = _torch()
    for t, name in ((cu_q, "cu_seqlens_q"), (cu_k, "cu_seqlens_k")):
        if t.dtype != torch.int32 or t.dim() != 1 or t.numel() < 2:
            raise ValueError(f"{name} must be a 1-D int32 tensor of nseq + 1 >= 2 offsets")
    if cu_k.numel() != cu_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    return cu_q.numel() - 1


def workspace_bytes(B, H, Nq, Nk, d, dtype_code, Hkv=None) -> int:
    """Workspace attn_fwd needs (nonzero only for Nq == 1); Hkv < H for grouped-query heads."""
    if Hkv is None or Hkv == H:
        return int(lib().attn_fwd_workspace_bytes(B, H, Nq, Nk, d, dtype_code))
    return int(lib().attn_fwd_gqa_workspace_bytes(B, H, Hkv, Nq, Nk, d, dtype_code))


def _dims(t, name, nd):
    if t.dim() != nd:
        raise ValueError(f"{name} must have {nd} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
             workspace=None, want_lse: bool = True):
    """O, LSE = attention(q, k, v) for [B, H, N, d] bf16/fp16 GPU tensors.
    k and v may have fewer heads than q (grouped-query attention: query head
    h reads K/V head h // (H // Hkv))."""
    torch = _torch()
    B, H, Nq, d = _dims(q, "q", 4)
    Hkv, Nk = _dims(k, "k", 4)[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != (B, Hkv, Nk, d):
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", numel=B * H * Nq, dtype=torch.float32)
    wsb = workspace_bytes(B, H, Nq, Nk, d, code, Hkv)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, device=q.device, dtype=torch.uint8)
    _need_workspace(workspace, wsb)
    args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(lse, "lse") if lse is not None else None]
    tail = [d, scale, int(bool(causal)), code, _dev(workspace, "workspace") if workspace is not None else None,
            _nbytes(workspace) if workspace is not None else 0, _stream()]
    if Hkv == H:
        rc = lib().attn_fwd(*args, B, H, Nq, Nk, *tail)
        _check(rc, "attn_fwd")
    else:
        rc = lib().attn_fwd_gqa(*args, B, H, Hkv, Nq, Nk, *tail)
        _check(rc, "attn_fwd_gqa")
    return out, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Packed variable-length batch: q [H, total_q, d], k, v [Hkv, total_k, d],
    cu_seqlens_* int32 GPU tensors of nseq + 1 offsets.  Returns (out, lse)
    with lse [H, total_q]."""
    torch = _torch()
    H, total_q, d = _dims(q, "q", 3)
    Hkv, total_k = _dims(k, "k", 3)[0], k.shape[1]
    if k.shape != (Hkv, total_k, d) or v.shape != (Hkv, total_k, d):
        raise ValueError("q must be [H, total_q, d] and k, v [Hkv, total_k, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    nseq = _need_offsets(cu_seqlens_q, cu_seqlens_k)
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else _need(out, "out", q.shape, q.dtype)
    lse = (torch.empty((H, total_q), device=q.device, dtype=torch.float32) if lse is None
           else _need(lse, "lse", numel=H * total_q, dtype=torch.float32))
    rc = lib().attn_fwd_varlen(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(lse, "lse"),
                               _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"), nseq,
                               int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, H, Hkv, d, scale,
                               int(bool(causal)), code, _stream())
    _check(rc, "attn_fwd_varlen")
    return out, lse


def attn_bwd(q, k, v, out, dout, lse, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
             workspace=None):
    """dQ, dK, dV of sum(dout * out) for out, lse = attn_fwd(q, k, v, causal, scale).
    k, v may have fewer heads than q (grouped-query attention)."""
    torch = _torch()
    B, H, Nq, d = _dims(q, "q", 4)
    Hkv, Nk = _dims(k, "k", 4)[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != (B, Hkv, Nk, d) or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, out, dout must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise ValueError("q, k, v, out, dout must share one dtype")
    if lse is None or lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be the [B, H, Nq] float32 log-sum-exp of the forward")
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else _need(dq, "dq", q.shape, q.dtype)
    dk = torch.empty_like(k) if dk is None else _need(dk, "dk", k.shape, k.dtype)
    dv = torch.empty_like(v) if dv is None else _need(dv, "dv", v.shape, v.dtype)
    wsb = int(lib().attn_bwd_workspace_bytes(B, H, Nq, Nk, d, code))
    if workspace is None:
        workspace = torch.empty(wsb, device=q.device, dtype=torch.uint8)
    _need_workspace(workspace, wsb)
    args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(dout, "dout"), _dev(lse, "lse"),
            _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv")]
    tail = [d, scale, int(bool(causal)), code, _dev(workspace, "workspace"), _nbytes(workspace), _stream()]
    if Hkv == H:
        _check(lib().attn_bwd(*args, B, H, Nq, Nk, *tail), "attn_bwd")
    else:
        _check(lib().attn_bwd_gqa(*args, B, H, Hkv, Nq, Nk, *tail), "attn_bwd_gqa")
    return dq, dk, dv


def attn_bwd_varlen(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients for attn_fwd_varlen (same packed layouts)."""
    torch = _torch()
    H, total_q, d = _dims(q, "q", 3)
    Hkv, total_k = _dims(k, "k", 3)[0], k.shape[1]
    if k.shape != (Hkv, total_k, d) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, out, dout must be [H, total_q, d] and k, v [Hkv, total_k, d]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise ValueError("q, k, v, out, dout must share one dtype")
    if lse is None or lse.shape != (H, total_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be the [H, total_q] float32 log-sum-exp of attn_fwd_varlen")
    nseq = _need_offsets(cu_seqlens_q, cu_seqlens_k)
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else _need(dq, "dq", q.shape, q.dtype)
    dk = torch.empty_like(k) if dk is None else _need(dk, "dk", k.shape, k.dtype)
    dv = torch.empty_like(v) if dv is None else _need(dv, "dv", v.shape, v.dtype)
    wsb = max(16, H * total_q * 8)
    if workspace is None:
        workspace = torch.empty(wsb, device=q.device, dtype=torch.uint8)
    _need_workspace(workspace, H * total_q * 8)
    rc = lib().attn_bwd_varlen(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(dout, "dout"),
                               _dev(lse, "lse"), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"),
                               _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"), nseq,
                               int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, H, Hkv, d, scale,
                               int(bool(causal)), code, _dev(workspace, "workspace"), _nbytes(workspace),
                               _stream())
    _check(rc, "attn_bwd_varlen")
    return dq, dk, dv


def decode_splits(B, H, Nk, d) -> int:
    return int(lib().attn_fwd_decode_splits(B, H, Nk, d))


def _decode_shapes(q, k, v, out, lse):
    """Shapes of a split-KV decode call: q, out [B, H, 1, d], k, v [B, H, Nk, d]."""
    torch = _torch()
    B, H, Nq, d = _dims(q, "q", 4)
    if Nq != 1:
        raise ValueError("decode takes one query per (batch, head)")
    Nk = _dims(k, "k", 4)[2]
    if k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] for q [B, H, 1, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    code = _dtype_code(q)
    out = torch.empty_like(q) if out is None else _need(out, "out", q.shape, q.dtype)
    lse = (torch.empty((B, H, 1), device=q.device, dtype=torch.float32) if lse is None
           else _need(lse, "lse", numel=B * H, dtype=torch.float32))
    return B, H, Nk, d, code, out, lse


def attn_fwd_decode(q, k, v, num_splits: int, scale: float | None = None, out=None, lse=None, workspace=None):
    """Split-KV decode: q [B, H, 1, d] against k, v [B, H, Nk, d]."""
    torch = _torch()
    B, H, Nk, d, code, out, lse = _decode_shapes(q, k, v, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    wsb = int(lib().attn_decode_workspace_bytes(B, H, d, num_splits))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), device=q.device, dtype=torch.uint8)
    _need_workspace(workspace, wsb)
    rc = lib().attn_fwd_decode(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(lse, "lse"),
                               B, H, Nk, d, scale, code, num_splits, _dev(workspace, "workspace"),
                               _nbytes(workspace), _stream())
    _check(rc, "attn_fwd_decode")
    return out, lse


def quantize_rows_i8(x):
    """Per-token int8 of a bf16 [..., d] tensor -> (int8 [..., d], fp32 scales [...])."""
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise ValueError("quantize_rows_i8 takes bf16")
    d = x.shape[-1]
    rows = x.numel() // d
    x8 = torch.empty(x.shape, device=x.device, dtype=torch.int8)
    s = torch.empty(x.shape[:-1], device=x.device, dtype=torch.float32)
    _check(lib().attn_quantize_rows_i8(_dev(x, "x"), _dev(x8, "x8"), _dev(s, "scales"), rows, d, _stream()),
           "attn_quantize_rows_i8")
    return x8, s


def quantize_tensor_e4m3(x, workspace=None):
    """Per-tensor E4M3 of a bf16 tensor -> (uint8 codes, fp32 scale as a 1-element GPU tensor)."""
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise ValueError("quantize_tensor_e4m3 takes bf16")
    n = x.numel()
    x8 = torch.empty(x.shape, device=x.device, dtype=torch.uint8)
    s = torch.empty(1, device=x.device, dtype=torch.float32)
    wsb = int(lib().attn_quantize_e4m3_workspace_bytes(n))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), device=x.device, dtype=torch.uint8)
    _need_workspace(workspace, wsb)
    _check(lib().attn_quantize_tensor_e4m3(_dev(x, "x"), _dev(x8, "x8"), _dev(s, "scale"), n,
                                           _dev(workspace, "workspace"), _nbytes(workspace), _stream()),
           "attn_quantize_tensor_e4m3")
    return x8, s


def _quant_shapes(q8, k8, v8, q_scale, k_scale, v_scale, qk_dtype, v_dtype, out, lse):
    """Shapes and dtypes of a quantised forward: q8 [B, H, Nq, d], k8, v8
    [B, H, Nk, d], q_scale B*H*Nq, k_scale B*H*Nk, v_scale one float32."""
    torch = _torch()
    B, H, Nq, d = _dims(q8, "q8", 4)
    Nk = _dims(k8, "k8", 4)[2]
    _need(q8, "q8", dtype=qk_dtype)
    _need(k8, "k8", (B, H, Nk, d), qk_dtype)
    _need(v8, "v8", (B, H, Nk, d), v_dtype)
    _need(q_scale, "q_scale", numel=B * H * Nq, dtype=torch.float32)
    _need(k_scale, "k_scale", numel=B * H * Nk, dtype=torch.float32)
    _need(v_scale, "v_scale", numel=1, dtype=torch.float32)
    out = (torch.empty((B, H, Nq, d), device=q8.device, dtype=torch.bfloat16) if out is None
           else _need(out, "out", (B, H, Nq, d), torch.bfloat16))
    lse = (torch.empty((B, H, Nq), device=q8.device, dtype=torch.float32) if lse is None
           else _need(lse, "lse", numel=B * H * Nq, dtype=torch.float32))
    return B, H, Nq, Nk, d, out, lse


def _quant_call(name, q8, k8, v8, q_scale, k_scale, v_scale, qk_dtype, v_dtype, causal, scale, out, lse):
    B, H, Nq, Nk, d, out, lse = _quant_shapes(q8, k8, v8, q_scale, k_scale, v_scale, qk_dtype, v_dtype, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = getattr(lib(), name)(_dev(q8, "q8"), _dev(k8, "k8"), _dev(v8, "v8"), _dev(q_scale, "q_scale"),
                              _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(out, "out"),
                              _dev(lse, "lse"), B, H, Nq, Nk, d, scale, int(bool(causal)), _stream())
    _check(rc, name)
    return out, lse


def attn_fwd_q8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None,
                out=None, lse=None):
    """Quantised forward: int8 q8/k8 [B,H,N,d] with per-token scales, E4M3 v8 with a
    per-tensor scale (1-element GPU tensor).  Returns (O bf16, LSE fp32)."""
    torch = _torch()
    return _quant_call("attn_fwd_q8", q8, k8, v8, q_scale, k_scale, v_scale, torch.int8, torch.uint8, causal,
                       scale, out, lse)


def quantize_tensor_i8(x, workspace=None):
    """Per-tensor int8 of a bf16 tensor -> (int8 codes, fp32 scale as a 1-element GPU tensor)."""
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise ValueError("quantize_tensor_i8 takes bf16")
    n = x.numel()
    x8 = torch.empty(x.shape, device=x.device, dtype=torch.int8)
    s = torch.empty(1, device=x.device, dtype=torch.float32)
    wsb = int(lib().attn_quantize_e4m3_workspace_bytes(n))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), device=x.device, dtype=torch.uint8)
    _need_workspace(workspace, wsb)
    _check(lib().attn_quantize_tensor_i8(_dev(x, "x"), _dev(x8, "x8"), _dev(s, "scale"), n,
                                         _dev(workspace, "workspace"), _nbytes(workspace), _stream()),
           "attn_quantize_tensor_i8")
    return x8, s


def attn_fwd_i8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None,
                out=None, lse=None):
    """All-INT8 forward: int8 q8/k8 [B,H,N,d] with per-token scales, int8 v8 with a
    per-tensor scale (1-element GPU tensor).  Returns (O bf16, LSE fp32)."""
    torch = _torch()
    return _quant_call("attn_fwd_i8", q8, k8, v8, q_scale, k_scale, v_scale, torch.int8, torch.int8, causal,
                       scale, out, lse)


def rotate_quantize_e4m3(x, signs=None, block_rows: int = 64):
    """Block E4M3 codes of a bf16 [..., N, d] tensor, rotated by diag(signs) H_d
    first when signs (a d-element float32 GPU tensor of +-1) is given ->
    (uint8 codes [..., N, d], fp32 per-row scales [..., N])."""
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise ValueError("rotate_quantize_e4m3 takes bf16")
    if x.dim() < 2:
        raise ValueError("rotate_quantize_e4m3 takes a [..., N, d] tensor")
    *lead, N, d = x.shape
    BH = int(math.prod(lead)) if lead else 1
    x8 = torch.empty(x.shape, device=x.device, dtype=torch.uint8)
    sc = torch.empty((*lead, N), device=x.device, dtype=torch.float32)
    sp = None
    if signs is not None:
        _need(signs, "signs", numel=d, dtype=torch.float32)
        sp = _dev(signs, "signs")
    _check(lib().attn_rotate_quantize_e4m3(_dev(x, "x"), sp, _dev(x8, "x8"), _dev(sc, "scales"), BH, N, d,
                                           int(block_rows), _stream()), "attn_rotate_quantize_e4m3")
    return x8, sc


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None,
                 out=None, lse=None):
    """FP8 forward: E4M3 q8/k8 [B,H,N,d] with per-row scales (from
    rotate_quantize_e4m3), E4M3 v8 with a per-tensor scale (1-element GPU
    tensor).  Returns (O bf16, LSE fp32)."""
    torch = _torch()
    return _quant_call("attn_fwd_fp8", q8, k8, v8, q_scale, k_scale, v_scale, torch.uint8, torch.uint8, causal,
                       scale, out, lse)


def attn_fwd_fp4p(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None,
                  out=None, lse=None):
    """attn_fwd_fp8 with P in MXFP4 (E2M1 codes, one power-of-two scale per 32
    keys of a query).  Same arguments and results as attn_fwd_fp8."""
    torch = _torch()
    return _quant_call("attn_fwd_fp4p", q8, k8, v8, q_scale, k_scale, v_scale, torch.uint8, torch.uint8, causal,
                       scale, out, lse)


def _debug_qk(name, q8, k8, code_dtype, out_dtype):
    torch = _torch()
    Nq, d = _dims(q8, "q8", 2)
    Nk = _dims(k8, "k8", 2)[0]
    _need(q8, "q8", dtype=code_dtype)
    _need(k8, "k8", (Nk, d), code_dtype)
    s = torch.empty((Nq, Nk), device=q8.device, dtype=out_dtype)
    _check(getattr(lib(), name)(_dev(q8, "q8"), _dev(k8, "k8"), _dev(s, "s"), Nq, Nk, d, _stream()), name)
    return s


def debug_qk_i32(q8, k8):
    """int32 Q8 K8^T of one head through the quantised kernel's tile routine."""
    torch = _torch()
    return _debug_qk("attn_debug_qk_i32", q8, k8, torch.int8, torch.int32)


def debug_qk_f8(q8, k8):
    """fp32 scores of one head's E4M3 codes through the fp8 kernel's tile routine."""
    torch = _torch()
    return _debug_qk("attn_debug_qk_f8", q8, k8, torch.uint8, torch.float32)


def debug_cvt_e2m1(x):
    """E2M1 codes (one per byte) of an fp32 GPU tensor through the library's FP4 conversion."""
    torch = _torch()
    _need(x, "x", dtype=torch.float32)
    y = torch.empty(x.shape, device=x.device, dtype=torch.uint8)
    _check(lib().attn_debug_cvt_e2m1(_dev(x, "x"), _dev(y, "y"), x.numel(), _stream()), "attn_debug_cvt_e2m1")
    return y


def debug_cvt_e4m3(x):
    """E4M3 codes of an fp32 GPU tensor through the library's conversion routine."""
    torch = _torch()
    _need(x, "x", dtype=torch.float32)
    y = torch.empty(x.shape, device=x.device, dtype=torch.uint8)
    _check(lib().attn_debug_cvt_e4m3(_dev(x, "x"), _dev(y, "y"), x.numel(), _stream()), "attn_debug_cvt_e4m3")
    return y


def attn_fwd_exp2_split(q, k, v, poly_per_8: int, causal: bool = False, scale: float | None = None, out=None,
                        lse=None):
    """The dense prefill with poly_per_8 (0, 2 or 4) of every 8 softmax
    exponentials on the library's polynomial exp2 (d = 128 for 2 and 4).
    q, k, v [B, H, N, d] bf16/fp16.  Returns (O, LSE)."""
    torch = _torch()
    B, H, Nq, d = _dims(q, "q", 4)
    Nk = _dims(k, "k", 4)[2]
    if k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d] of one dtype")
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else _need(out, "out", q.shape, q.dtype)
    lse = (torch.empty((B, H, Nq), device=q.device, dtype=torch.float32) if lse is None
           else _need(lse, "lse", numel=B * H * Nq, dtype=torch.float32))
    _check(lib().attn_fwd_exp2_split(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(lse, "lse"),
                                     B, H, Nq, Nk, d, scale, int(bool(causal)), code, int(poly_per_8),
                                     _stream()), "attn_fwd_exp2_split")
    return out, lse


def debug_exp2_poly(x):
    """The library's polynomial exp2 at every element of an fp32 GPU tensor."""
    torch = _torch()
    _need(x, "x", dtype=torch.float32)
    y = torch.empty(x.shape, device=x.device, dtype=torch.float32)
    _check(lib().attn_debug_exp2_poly(_dev(x, "x"), _dev(y, "y"), x.numel(), _stream()), "attn_debug_exp2_poly")
    return y

"""The Python binding checks every tensor's shape, dtype and size before it
takes a pointer (no GPU needed: these are CPU tensors, and every case fails
a check before the GPU-tensor check or any library call is reached)."""
import pytest
import torch

from flashattention_forward_amd import binding as Bd

bf, f16, f32, i8, u8, i32 = torch.bfloat16, torch.float16, torch.float32, torch.int8, torch.uint8, torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_fwd_checks():
    q, k, v = z(1, 2, 8, 64), z(1, 2, 16, 64), z(1, 2, 16, 64)
    raises(lambda: Bd.attn_fwd(q, z(1, 2, 16, 32), v), r"k, v \[B, Hkv, Nk, d\]")
    raises(lambda: Bd.attn_fwd(q, k, z(1, 2, 15, 64)), r"k, v \[B, Hkv, Nk, d\]")
    raises(lambda: Bd.attn_fwd(q, k, z(1, 2, 16, 64, dtype=f16)), "share one dtype")
    raises(lambda: Bd.attn_fwd(z(2, 8, 64), k, v), "4 dimensions")
    raises(lambda: Bd.attn_fwd(q, k, v, out=z(1, 2, 8, 32)), "out must have shape")
    raises(lambda: Bd.attn_fwd(q, k, v, out=z(1, 2, 8, 64, dtype=f16)), "out must be")
    raises(lambda: Bd.attn_fwd(q, k, v, out=z(1, 2, 8, 64), lse=z(1, 2, 7, dtype=f32)), "lse must hold 16")
    raises(lambda: Bd.attn_fwd(q, k, v, out=z(1, 2, 8, 64), lse=z(1, 2, 8, dtype=bf)), "lse must be")
    # decode: the workspace a caller brings must be large enough
    q1 = z(1, 2, 1, 64)
    raises(lambda: Bd.attn_fwd(q1, k, v, out=z(1, 2, 1, 64), lse=z(1, 2, 1, dtype=f32), workspace=z(4, dtype=u8)),
           "workspace holds 4 bytes")


def test_varlen_checks():
    q, k, v = z(2, 10, 64), z(1, 12, 64), z(1, 12, 64)
    cu = torch.tensor([0, 4, 10], dtype=i32)
    cuk = torch.tensor([0, 5, 12], dtype=i32)
    raises(lambda: Bd.attn_fwd_varlen(q, k, z(1, 11, 64), cu, cuk, 6, 7), r"k, v \[Hkv, total_k, d\]")
    raises(lambda: Bd.attn_fwd_varlen(q, k, v, cu.long(), cuk, 6, 7), "cu_seqlens_q must be a 1-D int32")
    raises(lambda: Bd.attn_fwd_varlen(q, k, v, cu, cuk[:2], 6, 7), "cu_seqlens_k must be a 1-D int32|same length")
    raises(lambda: Bd.attn_fwd_varlen(q, k, v, cu, torch.tensor([0, 12], dtype=i32), 6, 7), "same length")
    raises(lambda: Bd.attn_fwd_varlen(q, k, v, cu.view(1, 3), cuk, 6, 7), "cu_seqlens_q must be a 1-D int32")
    raises(lambda: Bd.attn_fwd_varlen(q, k, v, cu, cuk, 6, 7, out=z(2, 9, 64)), "out must have shape")
    raises(lambda: Bd.attn_fwd_varlen(q, k, v, cu, cuk, 6, 7, lse=z(2, 9, dtype=f32)), "lse must hold 20")
    raises(lambda: Bd.attn_fwd_varlen(q, k, z(1, 12, 64, dtype=f16), cu, cuk, 6, 7), "share one dtype")


def test_bwd_checks():
    q, k, v = z(1, 2, 8, 64), z(1, 2, 16, 64), z(1, 2, 16, 64)
    o, do, lse = z(1, 2, 8, 64), z(1, 2, 8, 64), z(1, 2, 8, dtype=f32)
    raises(lambda: Bd.attn_bwd(q, k, v, o, z(1, 2, 8, 32), lse), "q, out, dout must be")
    raises(lambda: Bd.attn_bwd(q, k, v, o, do, z(1, 2, 8, dtype=bf)), "lse must be")
    raises(lambda: Bd.attn_bwd(q, k, v, o, do, lse, dq=z(1, 2, 8, 32)), "dq must have shape")
    raises(lambda: Bd.attn_bwd(q, k, v, o, do, lse, dk=z(1, 2, 15, 64)), "dk must have shape")
    raises(lambda: Bd.attn_bwd(q, k, v, o, do, lse, dv=z(1, 2, 16, 64, dtype=f16)), "dv must be")
    raises(lambda: Bd.attn_bwd(q, k, v, o, do, lse, workspace=z(8, dtype=u8)), "workspace holds 8 bytes")
    raises(lambda: Bd.attn_bwd(q, k, v, o, z(1, 2, 8, 64, dtype=f16), lse), "share one dtype")


def test_bwd_varlen_checks():
    q, k, v = z(2, 10, 64), z(1, 12, 64), z(1, 12, 64)
    o, do, lse = z(2, 10, 64), z(2, 10, 64), z(2, 10, dtype=f32)
    cu, cuk = torch.tensor([0, 4, 10], dtype=i32), torch.tensor([0, 5, 12], dtype=i32)
    raises(lambda: Bd.attn_bwd_varlen(q, k, v, o, do, lse, cu.long(), cuk, 6, 7), "cu_seqlens_q must be")
    raises(lambda: Bd.attn_bwd_varlen(q, k, v, o, do, lse, cu, cuk[:2], 6, 7), "cu_seqlens_k must be|same length")
    raises(lambda: Bd.attn_bwd_varlen(q, k, v, o, do, z(2, 9, dtype=f32), cu, cuk, 6, 7), "lse must be")
    raises(lambda: Bd.attn_bwd_varlen(q, k, v, o, do, lse, cu, cuk, 6, 7, dk=z(1, 11, 64)), "dk must have shape")
    raises(lambda: Bd.attn_bwd_varlen(q, k, v, o, do, lse, cu, cuk, 6, 7, workspace=z(16, dtype=u8)),
           "workspace holds 16 bytes")


def test_decode_checks():
    q, k, v = z(2, 4, 1, 128), z(2, 4, 64, 128), z(2, 4, 64, 128)
    raises(lambda: Bd.attn_fwd_decode(z(2, 4, 2, 128), k, v, 2), "one query")
    raises(lambda: Bd.attn_fwd_decode(q, z(2, 4, 64, 64), v, 2), r"k and v must be \[B, H, Nk, d\]")
    raises(lambda: Bd.attn_fwd_decode(q, k, z(2, 2, 64, 128), 2), r"k and v must be \[B, H, Nk, d\]")
    raises(lambda: Bd.attn_fwd_decode(q, k, z(2, 4, 64, 128, dtype=f16), 2), "share one dtype")
    raises(lambda: Bd.attn_fwd_decode(q, k, v, 2, out=z(2, 4, 1, 64)), "out must have shape")
    raises(lambda: Bd.attn_fwd_decode(q, k, v, 2, lse=z(2, 3, 1, dtype=f32)), "lse must hold 8")
    raises(lambda: Bd.attn_fwd_decode(q, k, v, 2, workspace=z(64, dtype=u8)), "workspace holds 64 bytes")


@pytest.mark.parametrize("fn,qk,vt", [(Bd.attn_fwd_q8, i8, u8), (Bd.attn_fwd_i8, i8, i8),
                                      (Bd.attn_fwd_fp8, u8, u8), (Bd.attn_fwd_fp4p, u8, u8)])
def test_quantised_forward_checks(fn, qk, vt):
    B, H, Nq, Nk, d = 1, 2, 8, 16, 128
    q8, k8, v8 = z(B, H, Nq, d, dtype=qk), z(B, H, Nk, d, dtype=qk), z(B, H, Nk, d, dtype=vt)
    qs, ks, vs = z(B, H, Nq, dtype=f32), z(B, H, Nk, dtype=f32), z(1, dtype=f32)
    other = {i8: u8, u8: i8}
    raises(lambda: fn(q8.to(other[qk]), k8, v8, qs, ks, vs), "q8 must be")
    raises(lambda: fn(q8, k8[:, :, :15], v8, qs, ks, vs), "v8 must have shape")
    raises(lambda: fn(q8, k8, v8[:, :, :15], qs, ks, vs), "v8 must have shape")
    raises(lambda: fn(q8, k8, v8.to(other[vt]), qs, ks, vs), "v8 must be")
    raises(lambda: fn(q8, z(B, H, Nk, d, dtype=other[qk]), v8, qs, ks, vs), "k8 must be")
    raises(lambda: fn(q8, k8, v8, qs[:, :, :7], ks, vs), "q_scale must hold 16")
    raises(lambda: fn(q8, k8, v8, qs, ks[:, :, :15], vs), "k_scale must hold 32")
    raises(lambda: fn(q8, k8, v8, qs, ks, z(2, dtype=f32)), "v_scale must hold 1")
    raises(lambda: fn(q8, k8, v8, qs.to(bf), ks, vs), "q_scale must be")
    raises(lambda: fn(q8, k8, v8, qs, ks, vs, out=z(B, H, Nq, d, dtype=f16)), "out must be")
    raises(lambda: fn(q8, k8, v8, qs, ks, vs, out=z(B, H, Nq, 64)), "out must have shape")
    raises(lambda: fn(q8, k8, v8, qs, ks, vs, lse=z(B, H, 7, dtype=f32)), "lse must hold 16")
    raises(lambda: fn(q8[0], k8, v8, qs, ks, vs), "4 dimensions")


def test_debug_and_quantiser_checks():
    raises(lambda: Bd.debug_qk_i32(z(4, 128, dtype=u8), z(4, 128, dtype=i8)), "q8 must be")
    raises(lambda: Bd.debug_qk_i32(z(4, 128, dtype=i8), z(4, 64, dtype=i8)), "k8 must have shape")
    raises(lambda: Bd.debug_qk_f8(z(4, 128, dtype=u8), z(4, 128, dtype=i8)), "k8 must be")
    raises(lambda: Bd.debug_cvt_e4m3(z(8, dtype=f16)), "x must be")
    raises(lambda: Bd.debug_cvt_e2m1(z(8, dtype=bf)), "x must be")
    raises(lambda: Bd.debug_exp2_poly(z(8, dtype=torch.float64)), "x must be")
    raises(lambda: Bd.rotate_quantize_e4m3(z(4, 128), signs=z(64, dtype=f32)), "signs must hold 128")
    raises(lambda: Bd.rotate_quantize_e4m3(z(4, 128), signs=z(128, dtype=bf)), "signs must be")
    raises(lambda: Bd.quantize_tensor_e4m3(z(64), workspace=z(1, dtype=u8)), "workspace holds 1 bytes")
    raises(lambda: Bd.quantize_tensor_i8(z(64), workspace=z(1, dtype=u8)), "workspace holds 1 bytes")


def test_exp2_split_checks():
    q, k, v = z(1, 2, 8, 128), z(1, 2, 16, 128), z(1, 2, 16, 128)
    raises(lambda: Bd.attn_fwd_exp2_split(q, k, z(1, 2, 15, 128), 2), "one dtype")
    raises(lambda: Bd.attn_fwd_exp2_split(q, k, v, 2, out=z(1, 2, 8, 64)), "out must have shape")
    raises(lambda: Bd.attn_fwd_exp2_split(q, k, v, 2, lse=z(1, 2, 9, dtype=f32)), "lse must hold 16")


def test_well_formed_cpu_tensors_reach_the_device_check():
    """With every shape right, the only complaint left about CPU tensors is
    that they are not on the GPU (so the checks above are not over-strict)."""
    q, k, v = z(1, 2, 8, 64), z(1, 2, 16, 64), z(1, 2, 16, 64)
    raises(lambda: Bd.attn_fwd(q, k, v), "must be a GPU tensor")
    B, H, Nq, Nk, d = 1, 2, 8, 16, 128
    raises(lambda: Bd.attn_fwd_q8(z(B, H, Nq, d, dtype=i8), z(B, H, Nk, d, dtype=i8), z(B, H, Nk, d, dtype=u8),
                                  z(B, H, Nq, dtype=f32), z(B, H, Nk, dtype=f32), z(1, dtype=f32)),
           "must be a GPU tensor")

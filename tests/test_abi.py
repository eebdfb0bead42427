"""The C-ABI library: it loads, exports every declared symbol, and rejects
bad arguments before launching anything (no GPU needed: every call here
fails validation on the host)."""
import ctypes
import os
import re

import pytest

from flashattention_forward_amd import binding as Bd

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn_mi355x.h")
A = 0x10000          # a fake, 16-byte aligned address: never dereferenced (validation fails first)
MIS = 0x10008        # misaligned

# tests/test_abi_sanitized.py runs this file again against a CPU build of the
# same validation layer (api.cpp, plan.cpp) under AddressSanitizer and
# UndefinedBehaviorSanitizer, whose kernel launchers are stubs that only count
# launches; there the calls that pass every check run too (stub_only tests).
VALIDATION_LIB = os.environ.get("ATTN_VALIDATION_LIB")
if VALIDATION_LIB:
    Bd.LIB_PATH = VALIDATION_LIB
    Bd._lib = None
stub_only = pytest.mark.skipif(not VALIDATION_LIB, reason="an accepted call launches kernels: checked against the "
                                                           "stub launchers of the sanitizer build only")
SPAN_MAX = (1 << 31) - (1 << 16)   # largest head of Q, K, V or O in bytes (buffer-resource span)


def launches() -> int:
    return ctypes.CDLL(Bd.LIB_PATH).attn_stub_launches()


def accepted(call) -> bool:
    """The call passed validation and asked for exactly one launch sequence."""
    before = launches()
    rc = call()
    return rc == Bd.ATTN_OK and launches() > before


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_api():
    names = declared_functions()
    assert "attn_fwd" in names and "attn_fwd_q8" in names and len(names) == len(Bd.SIGNATURES)
    assert set(names) == set(Bd.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = Bd.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {Bd.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def fwd(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=1, Nq=4, Nk=4, d=64, scale=0.125, causal=0, dtype=0,
             ws=None, wsb=0)
    a.update(kw)
    return Bd.lib().attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                             a["scale"], a["causal"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), Bd.ATTN_E_INVALID), (dict(v=None), Bd.ATTN_E_INVALID), (dict(out=None), Bd.ATTN_E_INVALID),
    (dict(k=MIS), Bd.ATTN_E_INVALID), (dict(lse=A + 2), Bd.ATTN_E_INVALID),
    (dict(B=0), Bd.ATTN_E_INVALID), (dict(H=-1), Bd.ATTN_E_INVALID), (dict(Nq=0), Bd.ATTN_E_INVALID),
    (dict(Nk=0), Bd.ATTN_E_INVALID),
    (dict(scale=0.0), Bd.ATTN_E_INVALID), (dict(scale=-1.0), Bd.ATTN_E_INVALID),
    (dict(scale=float("nan")), Bd.ATTN_E_INVALID), (dict(scale=float("inf")), Bd.ATTN_E_INVALID),
    (dict(causal=1, Nq=5, Nk=4), Bd.ATTN_E_INVALID),
    (dict(B=2 ** 20, H=2 ** 20), Bd.ATTN_E_INVALID),
    # one head of K or Q past the buffer-resource span (2^31 - 2^16 bytes)
    (dict(Nk=2 ** 24, d=128), Bd.ATTN_E_INVALID), (dict(Nq=2 ** 25, Nk=2 ** 25, d=64), Bd.ATTN_E_INVALID),
    (dict(Nk=SPAN_MAX // 256 + 1, d=128), Bd.ATTN_E_INVALID),
    (dict(Nq=SPAN_MAX // 128 + 1, Nk=SPAN_MAX // 128 + 1, d=64), Bd.ATTN_E_INVALID),
    (dict(d=96), Bd.ATTN_E_UNSUPPORTED), (dict(d=256), Bd.ATTN_E_UNSUPPORTED), (dict(dtype=2), Bd.ATTN_E_UNSUPPORTED),
    (dict(Nq=1, ws=None, wsb=0), Bd.ATTN_E_WORKSPACE), (dict(Nq=1, ws=A, wsb=16), Bd.ATTN_E_WORKSPACE),
    (dict(Nq=1, ws=MIS, wsb=1 << 20), Bd.ATTN_E_WORKSPACE),
])
def test_attn_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def test_workspace_sizes():
    L = Bd.lib()
    assert L.attn_fwd_workspace_bytes(4, 32, 4096, 4096, 128, 0) == 0
    s = L.attn_fwd_decode_splits(64, 32, 8192, 128)
    assert 1 <= s <= 256
    assert L.attn_fwd_workspace_bytes(64, 32, 1, 8192, 128, 0) == 64 * 32 * s * 129 * 4
    assert L.attn_decode_workspace_bytes(2, 3, 64, 5) == 2 * 3 * 5 * 65 * 4
    assert L.attn_decode_workspace_bytes(2, 3, 96, 5) == 0
    assert L.attn_fwd_workspace_bytes(1, 1, 1, 1, 96, 0) == 0
    # small problems still split into several ranges only while each keeps >= 128 keys
    assert L.attn_fwd_decode_splits(1, 1, 100, 128) == 1


def test_decode_rejects():
    L = Bd.lib()
    args = lambda ns, ws, wsb, d=128, dt=0: L.attn_fwd_decode(A, A, A, A, A, 2, 2, 64, d, 0.1, dt, ns, ws, wsb, None)
    assert args(0, A, 1 << 20) == Bd.ATTN_E_INVALID
    assert args(65, A, 1 << 20) == Bd.ATTN_E_INVALID      # more splits than keys
    assert args(257, A, 1 << 20) == Bd.ATTN_E_INVALID
    assert args(4, None, 0) == Bd.ATTN_E_WORKSPACE
    assert args(4, A, L.attn_decode_workspace_bytes(2, 2, 128, 4) - 1) == Bd.ATTN_E_WORKSPACE
    assert args(4, A, 1 << 20, d=80) == Bd.ATTN_E_UNSUPPORTED
    assert args(4, A, 1 << 20, dt=7) == Bd.ATTN_E_UNSUPPORTED


def test_quant_entry_points_reject():
    L = Bd.lib()
    q8 = lambda **kw: L.attn_fwd_q8(kw.get("q", A), A, A, kw.get("qs", A), A, kw.get("vs", A), A, None, 1, 1,
                                    kw.get("Nq", 8), 8, kw.get("d", 128), kw.get("scale", 0.1),
                                    kw.get("causal", 0), None)
    assert q8(d=64) == Bd.ATTN_E_UNSUPPORTED
    assert q8(qs=None) == Bd.ATTN_E_INVALID
    assert q8(vs=None) == Bd.ATTN_E_INVALID
    assert q8(q=None) == Bd.ATTN_E_INVALID
    assert q8(Nq=9, causal=1) == Bd.ATTN_E_INVALID
    assert q8(scale=float("nan")) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_rows_i8(A, A, A, 10, 96, None) == Bd.ATTN_E_UNSUPPORTED
    assert L.attn_quantize_rows_i8(A, A, A, 0, 128, None) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_rows_i8(MIS, A, A, 4, 128, None) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_e4m3_workspace_bytes(12) == 0
    assert L.attn_quantize_e4m3_workspace_bytes(1 << 20) > 0
    assert L.attn_quantize_tensor_e4m3(A, A, A, 12, A, 4096, None) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_tensor_e4m3(A, A, A, 1 << 20, A, 4, None) == Bd.ATTN_E_WORKSPACE
    assert L.attn_quantize_tensor_e4m3(A, A, A, 1 << 20, None, 1 << 20, None) == Bd.ATTN_E_WORKSPACE
    i8 = lambda **kw: L.attn_fwd_i8(kw.get("q", A), A, kw.get("v", A), A, kw.get("ks", A), kw.get("vs", A), A, A,
                                    1, 1, kw.get("Nq", 8), 8, kw.get("d", 128), kw.get("scale", 0.1),
                                    kw.get("causal", 0), None)
    assert i8(d=64) == Bd.ATTN_E_UNSUPPORTED
    assert i8(ks=None) == Bd.ATTN_E_INVALID
    assert i8(vs=None) == Bd.ATTN_E_INVALID
    assert i8(vs=A + 2) == Bd.ATTN_E_INVALID  # scale pointers need 4-byte alignment
    assert i8(v=None) == Bd.ATTN_E_INVALID
    assert i8(Nq=9, causal=1) == Bd.ATTN_E_INVALID
    assert i8(scale=float("inf")) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_tensor_i8(A, A, A, 12, A, 4096, None) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_tensor_i8(A, A, A, 0, A, 4096, None) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_tensor_i8(MIS, A, A, 1 << 20, A, 1 << 20, None) == Bd.ATTN_E_INVALID
    assert L.attn_quantize_tensor_i8(A, A, A, 1 << 20, A, 4, None) == Bd.ATTN_E_WORKSPACE
    assert L.attn_quantize_tensor_i8(A, A, A, 1 << 20, None, 1 << 20, None) == Bd.ATTN_E_WORKSPACE
    f8 = lambda **kw: L.attn_fwd_fp8(kw.get("q", A), A, A, A, kw.get("ks", A), kw.get("vs", A), A, A,
                                     1, 1, kw.get("Nq", 8), 8, kw.get("d", 128), kw.get("scale", 0.1),
                                     kw.get("causal", 0), None)
    assert f8(d=64) == Bd.ATTN_E_UNSUPPORTED
    assert f8(ks=None) == Bd.ATTN_E_INVALID
    assert f8(vs=A + 2) == Bd.ATTN_E_INVALID
    assert f8(q=MIS) == Bd.ATTN_E_INVALID
    assert f8(Nq=9, causal=1) == Bd.ATTN_E_INVALID
    assert f8(scale=float("nan")) == Bd.ATTN_E_INVALID
    f4 = lambda **kw: L.attn_fwd_fp4p(kw.get("q", A), A, A, A, kw.get("ks", A), kw.get("vs", A), A, A,
                                      1, 1, kw.get("Nq", 8), 8, kw.get("d", 128), kw.get("scale", 0.1),
                                      kw.get("causal", 0), None)
    assert f4(d=64) == Bd.ATTN_E_UNSUPPORTED
    assert f4(ks=None) == Bd.ATTN_E_INVALID
    assert f4(vs=A + 2) == Bd.ATTN_E_INVALID
    assert f4(q=MIS) == Bd.ATTN_E_INVALID
    assert f4(Nq=9, causal=1) == Bd.ATTN_E_INVALID
    assert f4(scale=0.0) == Bd.ATTN_E_INVALID
    assert L.attn_debug_cvt_e2m1(A, A, 3, None) == Bd.ATTN_E_INVALID
    assert L.attn_debug_cvt_e2m1(A + 2, A, 4, None) == Bd.ATTN_E_INVALID
    rq = lambda **kw: L.attn_rotate_quantize_e4m3(kw.get("x", A), kw.get("signs", A), A, kw.get("sc", A),
                                                  kw.get("BH", 2), kw.get("N", 64), kw.get("d", 128),
                                                  kw.get("blk", 64), None)
    assert rq(d=64) == Bd.ATTN_E_UNSUPPORTED
    assert rq(signs=None, d=96) == Bd.ATTN_E_UNSUPPORTED
    assert rq(x=None) == Bd.ATTN_E_INVALID
    assert rq(x=MIS) == Bd.ATTN_E_INVALID
    assert rq(signs=A + 2) == Bd.ATTN_E_INVALID
    assert rq(sc=None) == Bd.ATTN_E_INVALID
    assert rq(BH=0) == Bd.ATTN_E_INVALID
    assert rq(N=0) == Bd.ATTN_E_INVALID
    assert rq(blk=0) == Bd.ATTN_E_INVALID
    assert L.attn_debug_qk_i32(A, A, A, 4, 4, 64, None) == Bd.ATTN_E_UNSUPPORTED
    assert L.attn_debug_qk_f8(A, A, A, 4, 4, 64, None) == Bd.ATTN_E_UNSUPPORTED
    assert L.attn_debug_qk_f8(A, None, A, 4, 4, 128, None) == Bd.ATTN_E_INVALID
    assert L.attn_debug_qk_i32(None, A, A, 4, 4, 128, None) == Bd.ATTN_E_INVALID
    assert L.attn_debug_cvt_e4m3(A, A, 3, None) == Bd.ATTN_E_INVALID


def bwd(**kw):
    a = dict(q=A, k=A, v=A, out=A, do=A, lse=A, dq=A, dk=A, dv=A, B=2, H=3, Nq=40, Nk=50, d=128, scale=0.1,
             causal=0, dtype=0, ws=A, wsb=1 << 20)
    a.update(kw)
    return Bd.lib().attn_bwd(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                             a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["ws"], a["wsb"],
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), Bd.ATTN_E_INVALID), (dict(do=None), Bd.ATTN_E_INVALID), (dict(lse=None), Bd.ATTN_E_INVALID),
    (dict(dq=None), Bd.ATTN_E_INVALID), (dict(dk=None), Bd.ATTN_E_INVALID), (dict(dv=None), Bd.ATTN_E_INVALID),
    (dict(do=MIS), Bd.ATTN_E_INVALID), (dict(dv=MIS), Bd.ATTN_E_INVALID), (dict(lse=A + 2), Bd.ATTN_E_INVALID),
    (dict(B=0), Bd.ATTN_E_INVALID), (dict(Nk=0), Bd.ATTN_E_INVALID), (dict(scale=0.0), Bd.ATTN_E_INVALID),
    (dict(causal=1, Nq=51), Bd.ATTN_E_INVALID), (dict(Nk=2 ** 24), Bd.ATTN_E_INVALID),
    (dict(d=96), Bd.ATTN_E_UNSUPPORTED), (dict(dtype=3), Bd.ATTN_E_UNSUPPORTED),
    (dict(ws=None), Bd.ATTN_E_WORKSPACE), (dict(wsb=2 * 3 * 40 * 8 - 1), Bd.ATTN_E_WORKSPACE),
    (dict(ws=MIS), Bd.ATTN_E_WORKSPACE),
])
def test_attn_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_size():
    L = Bd.lib()
    assert L.attn_bwd_workspace_bytes(4, 32, 4096, 4096, 128, 0) == 4 * 32 * 4096 * 8
    assert L.attn_bwd_workspace_bytes(0, 1, 1, 1, 64, 0) == 0


def test_gqa_and_varlen_reject():
    L = Bd.lib()
    gqa = lambda **kw: L.attn_fwd_gqa(A, A, A, A, A, 1, kw.get("H", 8), kw.get("Hkv", 2), kw.get("Nq", 16), 16,
                                      kw.get("d", 128), 0.1, 0, 0, None, 0, None)
    assert gqa(Hkv=3) == Bd.ATTN_E_INVALID          # H not a multiple of Hkv
    assert gqa(Hkv=0) == Bd.ATTN_E_INVALID
    assert gqa(d=80) == Bd.ATTN_E_UNSUPPORTED
    assert gqa(Nq=1) == Bd.ATTN_E_WORKSPACE           # decode needs its workspace
    s = L.attn_fwd_decode_splits(64, 32, 8192, 128)
    assert s == 2                                     # 4096 (head, key range) streams, >= 128 keys each
    assert L.attn_fwd_gqa_workspace_bytes(64, 32, 8, 1, 8192, 128, 0) == 64 * 32 * s * 129 * 4
    assert L.attn_fwd_gqa_workspace_bytes(64, 32, 32, 1, 8192, 128, 0) == L.attn_fwd_workspace_bytes(
        64, 32, 1, 8192, 128, 0)
    assert L.attn_fwd_gqa_workspace_bytes(1, 6, 4, 1, 100, 128, 0) == 0      # H not a multiple of Hkv
    assert L.attn_fwd_gqa_workspace_bytes(1, 8, 2, 5, 100, 128, 0) == 0      # prefill needs none
    vl = lambda **kw: L.attn_fwd_varlen(A, A, A, A, A, kw.get("cq", A), kw.get("ck", A), kw.get("nseq", 3),
                                        kw.get("mq", 100), kw.get("mk", 100), 300, 300, kw.get("H", 4),
                                        kw.get("Hkv", 2), kw.get("d", 64), kw.get("scale", 0.1), 0, 0, None)
    assert vl(cq=None) == Bd.ATTN_E_INVALID and vl(ck=None) == Bd.ATTN_E_INVALID
    assert vl(cq=A + 2) == Bd.ATTN_E_INVALID
    assert vl(nseq=0) == Bd.ATTN_E_INVALID and vl(Hkv=3) == Bd.ATTN_E_INVALID
    assert vl(mq=-1) == Bd.ATTN_E_INVALID and vl(scale=0.0) == Bd.ATTN_E_INVALID
    assert vl(mk=2 ** 25) == Bd.ATTN_E_INVALID       # one sequence's keys past the span limit
    assert vl(mk=SPAN_MAX // 128 + 1) == Bd.ATTN_E_INVALID
    assert vl(d=96) == Bd.ATTN_E_UNSUPPORTED
    assert vl(mq=0) == Bd.ATTN_OK                      # no query: nothing launched
    bg = lambda **kw: L.attn_bwd_gqa(A, A, A, A, A, A, A, A, A, 1, kw.get("H", 8), kw.get("Hkv", 2), 16, 16, 128,
                                     0.1, 0, 0, kw.get("ws", A), kw.get("wsb", 1 << 20), None)
    assert bg(Hkv=3) == Bd.ATTN_E_INVALID and bg(ws=None) == Bd.ATTN_E_WORKSPACE
    assert bg(wsb=8 * 16 * 8 - 1) == Bd.ATTN_E_WORKSPACE
    bv = lambda **kw: L.attn_bwd_varlen(A, A, A, A, A, A, A, A, A, kw.get("cq", A), A, 2, 50, 50, 100, 100,
                                        kw.get("H", 4), 2, 64, 0.1, 0, 0, kw.get("ws", A), kw.get("wsb", 1 << 20),
                                        None)
    assert bv(cq=None) == Bd.ATTN_E_INVALID and bv(H=3) == Bd.ATTN_E_INVALID
    assert bv(wsb=4 * 100 * 8 - 1) == Bd.ATTN_E_WORKSPACE and bv(ws=MIS) == Bd.ATTN_E_WORKSPACE


def test_status_strings_and_build_info():
    for c in (0, -1, -2, -3, -4):
        assert Bd.status_str(c) and Bd.status_str(c) != "unknown status"
    assert Bd.status_str(99) == "unknown status"
    assert "gfx950" in Bd.build_info()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(Bd, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(Bd, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        Bd.lib()


def test_exp2_split_rejects():
    """The software-exp2 split prefill: shares other than 0, 2, 4 are invalid;
    shares 2 and 4 need d = 128; otherwise attn_fwd's checks apply."""
    L = Bd.lib()
    sp = lambda **kw: L.attn_fwd_exp2_split(kw.get("q", A), A, A, A, kw.get("lse", A), 1, 1, kw.get("Nq", 8), 8,
                                            kw.get("d", 128), kw.get("scale", 0.1), kw.get("causal", 0),
                                            kw.get("dtype", Bd.ATTN_BF16), kw.get("poly", 2), None)
    assert sp(poly=3) == Bd.ATTN_E_INVALID
    assert sp(poly=8) == Bd.ATTN_E_INVALID
    assert sp(poly=-2) == Bd.ATTN_E_INVALID
    assert sp(d=64) == Bd.ATTN_E_UNSUPPORTED
    assert sp(d=96, poly=0) == Bd.ATTN_E_UNSUPPORTED
    assert sp(dtype=5) == Bd.ATTN_E_UNSUPPORTED
    assert sp(q=MIS) == Bd.ATTN_E_INVALID
    assert sp(lse=A + 2) == Bd.ATTN_E_INVALID
    assert sp(Nq=9, causal=1) == Bd.ATTN_E_INVALID
    assert sp(scale=float("nan")) == Bd.ATTN_E_INVALID
    assert L.attn_debug_exp2_poly(A, A, 0, None) == Bd.ATTN_E_INVALID
    assert L.attn_debug_exp2_poly(None, A, 8, None) == Bd.ATTN_E_INVALID
    assert L.attn_debug_exp2_poly(A + 2, A, 8, None) == Bd.ATTN_E_INVALID


@stub_only
def test_span_limit_both_sides():
    """Heads of exactly SPAN_MAX bytes are accepted, one row more is rejected:
    the bound the kernels' buffer resources are sized for (every offset they
    form, a prefetched tile past the end included, stays below 2^31)."""
    L = Bd.lib()
    for d in (64, 128):
        n = SPAN_MAX // (2 * d)
        assert n * 2 * d == SPAN_MAX
        assert accepted(lambda: fwd(Nq=8, Nk=n, d=d))
        assert fwd(Nq=8, Nk=n + 1, d=d) == Bd.ATTN_E_INVALID
        assert accepted(lambda: fwd(Nq=n, Nk=n, d=d, causal=1))
        assert fwd(Nq=n + 1, Nk=n + 1, d=d) == Bd.ATTN_E_INVALID
        assert accepted(lambda: bwd(B=1, H=1, Nq=8, Nk=n, d=d))
        assert bwd(B=1, H=1, Nq=8, Nk=n + 1, d=d) == Bd.ATTN_E_INVALID
        vl = lambda mk: L.attn_fwd_varlen(A, A, A, A, A, A, A, 2, 64, mk, 128, 2 * mk, 4, 2, d, 0.1, 0, 0, None)
        assert accepted(lambda: vl(n))
        assert vl(n + 1) == Bd.ATTN_E_INVALID


@stub_only
def test_valid_calls_launch():
    """Every entry point launches once its arguments pass, and never when
    they fail (a rejected call leaves the launch count unchanged)."""
    L = Bd.lib()
    assert accepted(lambda: fwd())
    assert accepted(lambda: fwd(Nq=1, ws=A, wsb=1 << 20))
    assert accepted(lambda: bwd())
    assert accepted(lambda: L.attn_fwd_gqa(A, A, A, A, A, 1, 8, 2, 16, 16, 128, 0.1, 1, 0, None, 0, None))
    assert accepted(lambda: L.attn_fwd_q8(A, A, A, A, A, A, A, None, 1, 2, 8, 8, 128, 0.1, 0, None))
    assert accepted(lambda: L.attn_quantize_tensor_e4m3(A, A, A, 1 << 20, A, 1 << 20, None))
    assert accepted(lambda: L.attn_rotate_quantize_e4m3(A, A, A, A, 2, 64, 128, 64, None))
    assert accepted(lambda: L.attn_fwd_exp2_split(A, A, A, A, A, 1, 1, 8, 8, 128, 0.1, 0, 0, 2, None))
    before = launches()
    assert fwd(d=96) == Bd.ATTN_E_UNSUPPORTED and bwd(ws=None) == Bd.ATTN_E_WORKSPACE
    assert L.attn_fwd_q8(A, A, A, None, A, A, A, None, 1, 2, 8, 8, 128, 0.1, 0, None) == Bd.ATTN_E_INVALID
    assert launches() == before


def test_static_decode_rejects():
    """attn_fwd_decode_static: attn_fwd_decode's checks, and partials larger
    than the static scratch (8 MiB) refused before any launch."""
    L = Bd.lib()
    st = lambda B=2, H=2, Nk=64, d=128, ns=4, dt=0, q=A: L.attn_fwd_decode_static(q, A, A, A, A, B, H, Nk, d, 0.1,
                                                                                   dt, ns, None)
    assert st(ns=0) == Bd.ATTN_E_INVALID and st(ns=65) == Bd.ATTN_E_INVALID and st(q=None) == Bd.ATTN_E_INVALID
    assert st(d=80) == Bd.ATTN_E_UNSUPPORTED and st(dt=7) == Bd.ATTN_E_UNSUPPORTED
    assert 64 * 32 * 16 * 129 * 4 > 8 << 20
    assert st(B=64, H=32, Nk=4096, ns=16) == Bd.ATTN_E_WORKSPACE


@stub_only
def test_static_decode_scratch_limit_both_sides():
    """Partials of exactly 8 MiB fit the static scratch; one split more does not."""
    L = Bd.lib()
    # B*H*splits*(d+1)*4 bytes: 16*32*16*(127+1)... with d = 128: 129 floats per (head, split)
    B, H, d = 1, 1, 128
    fit = (8 << 20) // ((d + 1) * 4)            # (head, split) slots that fit
    H = 254                                       # 254 heads x splits slots
    s = fit // H                                  # largest split count that fits
    assert H * s * (d + 1) * 4 <= 8 << 20 < H * (s + 1) * (d + 1) * 4
    call = lambda ns: L.attn_fwd_decode_static(A, A, A, A, A, B, H, 1 << 16, d, 0.1, 0, ns, None)
    assert accepted(lambda: call(s))
    assert call(s + 1) == Bd.ATTN_E_WORKSPACE

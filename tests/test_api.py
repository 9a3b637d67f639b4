"""The C ABI without a GPU: the library loads, exports what include/fa.h declares, and validates arguments.

Only calls that must fail validation are made here (validation runs before
any HIP call), with dummy but aligned pointer values that are never
dereferenced.
"""
import ctypes
import math
import os
import re

import pytest

from tiled_online_softmax_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x10000  # aligned dummy pointer, never dereferenced (validation fails first)


def header_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(fa.EXPORTED), names
    L = fa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert fa.status_string(fa.FA_OK) == "FA_OK"
    assert fa.status_string(fa.FA_ERR_WORKSPACE) == "FA_ERR_WORKSPACE"
    assert fa.status_string(99) == "FA_UNKNOWN_STATUS"


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, D=64, causal=0, scale=0.125, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.lib().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"], a["causal"],
                           a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG, "NULL"),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG, "NULL"),
    (dict(v=P + 8), fa.FA_ERR_INVALID_ARG, "aligned"),
    (dict(N=0), fa.FA_ERR_INVALID_ARG, ">= 1"),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG, ">= 1"),
    (dict(D=0), fa.FA_ERR_INVALID_ARG, ">= 1"),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG, "causal"),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARG, "scale"),
    (dict(scale=math.inf), fa.FA_ERR_INVALID_ARG, "scale"),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG, "scale"),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG, "scale"),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG, "dtype"),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED, "D=96"),
    (dict(D=512, dtype=fa.FA_FP8_E4M3), fa.FA_ERR_UNSUPPORTED, "D=512"),
    (dict(N=1 << 24, D=128), fa.FA_ERR_INVALID_ARG, "2^31"),
])
def test_fwd_validation(kw, status, msg):
    assert _fwd(**kw) == status
    assert msg in fa.last_error()


def test_fwd_ex_threshold_validation():
    L = fa.lib()
    for bad in (-1.0, math.nan, math.inf):
        assert L.fa_fwd_ex(P, P, P, P, P, 1, 1, 16, 64, 0, 0.1, fa.FA_BF16, bad, None) == fa.FA_ERR_INVALID_ARG
        assert "threshold" in fa.last_error()


def test_fwd_fp8_validation():
    L = fa.lib()
    assert L.fa_fwd_fp8(P, P, P, P, P, 1, 1, 16, 128, 0, 0.1, P + 2, None, None, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_fp8(P, P, P, P, P, 1, 1, 16, 192, 0, 0.1, None, None, None, None) == fa.FA_ERR_UNSUPPORTED


def test_fwd_fp8_general_and_varlen_validation():
    L = fa.lib()
    # fa_fwd_fp8_general(q, k, v, o, lse, B, H, Hkv, Nq, Nk, D, causal, window, scale, q_ds, k_ds, v_ds, stream)
    gen = lambda H=8, Hkv=2, Nq=16, Nk=32, D=128, window=-1, qd=None: L.fa_fwd_fp8_general(
        P, P, P, P, P, 1, H, Hkv, Nq, Nk, D, 1, window, 0.1, qd, None, None, None)
    assert gen(qd=P + 2) == fa.FA_ERR_INVALID_ARG and "descale" in fa.last_error()
    assert gen(Hkv=3) == fa.FA_ERR_INVALID_ARG and "divide" in fa.last_error()
    assert gen(Nk=0) == fa.FA_ERR_INVALID_ARG
    assert gen(window=-2) == fa.FA_ERR_INVALID_ARG
    assert gen(D=96) == fa.FA_ERR_UNSUPPORTED and "D=96" in fa.last_error()
    # fa_fwd_fp8_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, Hkv, Tq, Tk, max_q, max_k, D, causal, window, scale, ...)
    var = lambda cu=P, Tq=100, D=64, vd=None: L.fa_fwd_fp8_varlen(
        P, P, P, P, P, cu, P, 2, 4, 2, Tq, 100, 64, 64, D, 1, -1, 0.1, None, None, vd, None)
    assert var(cu=None) == fa.FA_ERR_INVALID_ARG and "cu_seqlens_q" in fa.last_error()
    assert var(vd=P + 1) == fa.FA_ERR_INVALID_ARG and "descale" in fa.last_error()
    assert var(Tq=0) == fa.FA_ERR_INVALID_ARG
    assert var(D=80) == fa.FA_ERR_UNSUPPORTED


def test_quantize_validation():
    L = fa.lib()
    assert L.fa_quantize_fp8(P, 0, P, P, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_quantize_fp8(None, 10, P, P, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_quantize_fp8(P, 10, P, None, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_quantize_fp8(P, 10, P, P + 1, None) == fa.FA_ERR_INVALID_ARG


def test_workspace_size():
    L = fa.lib()
    B, H, N, D = 2, 3, 100, 64
    det = L.fa_bwd_workspace_size(B, H, N, D, fa.FA_BF16, fa.FA_BWD_DETERMINISTIC)
    atom = L.fa_bwd_workspace_size(B, H, N, D, fa.FA_BF16, fa.FA_BWD_ATOMIC)
    assert det >= B * H * N * 8 and det % 256 == 0
    assert atom == det + B * H * N * D * 4
    assert L.fa_bwd_workspace_size(B, H, N, D, fa.FA_F32, 0) == 0
    assert L.fa_bwd_workspace_size(0, H, N, D, fa.FA_BF16, 0) == 0
    assert L.fa_bwd_workspace_size(B, H, N, D, fa.FA_BF16, 5) == 0


def _bwd(**kw):
    a = dict(B=1, H=1, N=16, D=64, causal=0, scale=0.125, dtype=fa.FA_BF16, variant=fa.FA_BWD_ATOMIC,
             ws=P, ws_bytes=1 << 20, ptr=P)
    a.update(kw)
    p = a["ptr"]
    return fa.lib().fa_bwd(P, P, P, P, P, P, p, P, P, a["B"], a["H"], a["N"], a["D"], a["causal"], a["scale"],
                           a["dtype"], a["variant"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=9), fa.FA_ERR_INVALID_ARG),
    (dict(variant=3), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),
    (dict(ptr=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
])
def test_bwd_validation(kw, status):
    assert _bwd(**kw) == status
    assert fa.last_error() != ""


def test_error_string_is_per_thread():
    import threading

    _fwd(N=0)
    seen = {}

    def other():
        seen["msg"] = fa.last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert fa.last_error() != ""


def test_bwd_dkdv_validation():
    L = fa.lib()
    args = [P] * 8 + [1, 1, 16, 64, 0, 0.125]
    assert L.fa_bwd_dkdv(*args, fa.FA_F32, P, 1 << 20, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_bwd_dkdv(*args, fa.FA_BF16, None, 1 << 20, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_dkdv(*args, fa.FA_BF16, P, 8, None) == fa.FA_ERR_WORKSPACE
    bad = [P] * 7 + [None] + [1, 1, 16, 64, 0, 0.125]
    assert L.fa_bwd_dkdv(*bad, fa.FA_BF16, P, 1 << 20, None) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("H,Hkv,status,msg", [
    (8, 3, fa.FA_ERR_INVALID_ARG, "divide"),
    (8, 0, fa.FA_ERR_INVALID_ARG, "divide"),
    (4, 8, fa.FA_ERR_INVALID_ARG, "divide"),
    (8, -2, fa.FA_ERR_INVALID_ARG, "divide"),
])
def test_fwd_gqa_head_validation(H, Hkv, status, msg):
    L = fa.lib()
    assert L.fa_fwd_gqa(P, P, P, P, P, 1, H, Hkv, 16, 64, 0, 0.1, fa.FA_BF16, None) == status
    assert msg in fa.last_error()


def test_fwd_gqa_common_validation():
    L = fa.lib()
    assert L.fa_fwd_gqa(None, P, P, P, P, 1, 8, 2, 16, 64, 0, 0.1, fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_fwd_gqa(P, P, P, P, P, 1, 8, 2, 16, 96, 0, 0.1, fa.FA_BF16, None) == fa.FA_ERR_UNSUPPORTED


def test_bwd_gqa_validation():
    L = fa.lib()
    ws = fa.bwd_workspace_size(1, 8, 16, 64, fa.FA_BWD_DETERMINISTIC)

    def call(H, Hkv, N=16, D=64, variant=fa.FA_BWD_DETERMINISTIC, wsb=ws):
        return L.fa_bwd_gqa(P, P, P, P, P, P, P, P, P, 1, H, Hkv, N, D, 0, 0.1, fa.FA_BF16, variant, P, wsb, None)

    assert call(8, 3) == fa.FA_ERR_INVALID_ARG and "divide" in fa.last_error()
    assert call(8, 0) == fa.FA_ERR_INVALID_ARG
    assert call(8, 2, variant=2) == fa.FA_ERR_INVALID_ARG and "variant" in fa.last_error()
    assert call(8, 2, wsb=ws - 1) == fa.FA_ERR_WORKSPACE
    # 64 query heads of 2^20 x 64 bf16 (2^27 bytes each) share one K/V head: the group spans 2^33 bytes
    big = fa.bwd_workspace_size(1, 64, 1 << 20, 64, fa.FA_BWD_DETERMINISTIC)
    assert call(64, 1, N=1 << 20, wsb=big) == fa.FA_ERR_UNSUPPORTED and "2^31" in fa.last_error()


def _fwd_general(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Hkv=1, Nq=16, Nk=32, D=64, causal=1, window=-1, scale=0.125,
             dtype=fa.FA_BF16)
    a.update(kw)
    return fa.lib().fa_fwd_general(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Nq"],
                                   a["Nk"], a["D"], a["causal"], a["window"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG, "Nk"),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG, ">= 1"),
    (dict(window=-2), fa.FA_ERR_INVALID_ARG, "window"),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG, "divide"),
    (dict(Nk=1 << 24, D=128, Nq=16), fa.FA_ERR_UNSUPPORTED, "2^31"),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED, "D=96"),
    (dict(k=None), fa.FA_ERR_INVALID_ARG, "NULL"),
])
def test_fwd_general_validation(kw, status, msg):
    assert _fwd_general(**kw) == status
    assert msg in fa.last_error()


def test_bwd_general_validation():
    L = fa.lib()
    ws = fa.bwd_workspace_size(1, 2, 16, 64, fa.FA_BWD_DETERMINISTIC)

    def call(Nq=16, Nk=32, causal=1, window=-1, variant=fa.FA_BWD_DETERMINISTIC, wsb=ws, dtype=fa.FA_BF16):
        return L.fa_bwd_general(P, P, P, P, P, P, P, P, P, 1, 2, 1, Nq, Nk, 64, causal, window, 0.1, dtype, variant,
                                P, wsb, None)

    assert call(window=-5) == fa.FA_ERR_INVALID_ARG and "window" in fa.last_error()
    assert call(Nk=0) == fa.FA_ERR_INVALID_ARG
    assert call(variant=2) == fa.FA_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == fa.FA_ERR_WORKSPACE
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED


def test_binding_argument_counts_match_header():
    """Every ctypes prototype in the binding has as many arguments as the declaration in include/fa.h."""
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    L = fa.lib()
    for name, params in re.findall(r"\b(fa_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        n = 0 if params in ("", "void") else len(params.split(","))
        assert len(getattr(L, name).argtypes) == n, (name, n, len(getattr(L, name).argtypes))


def _fwd_strided(strides=None, **kw):
    a = dict(B=2, H=4, Hkv=2, Nq=16, Nk=32, D=64, causal=1, window=-1, scale=0.125, dtype=fa.FA_BF16)
    a.update(kw)
    B, H, Hkv, Nq, Nk, D = a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["D"]
    if strides is None:  # [B, N, H, D] views
        strides = [Nq * H * D, D, H * D, Nk * Hkv * D, D, Hkv * D, Nk * Hkv * D, D, Hkv * D, Nq * H * D, D, H * D,
                   H * Nq, Nq]
    arr = None if strides == "null" else (ctypes.c_longlong * 14)(*strides)
    return fa.lib().fa_fwd_strided(P, P, P, P, P, B, H, Hkv, Nq, Nk, D, a["causal"], a["window"], a["scale"],
                                   a["dtype"], arr, None)


def _bnhd(B, H, Hkv, Nq, Nk, D):
    q = [Nq * H * D, D, H * D]
    k = [Nk * Hkv * D, D, Hkv * D]
    return q, k


@pytest.mark.parametrize("edit,status,msg", [
    ("null", fa.FA_ERR_INVALID_ARG, "strides is NULL"),
    ({0: -1}, fa.FA_ERR_INVALID_ARG, "q strides"),
    ({5: 63}, fa.FA_ERR_INVALID_ARG, "row stride >= D"),
    ({2: 260}, fa.FA_ERR_INVALID_ARG, "16 bytes"),      # q rows 520 bytes apart
    ({4: 68}, fa.FA_ERR_INVALID_ARG, "16 bytes"),       # k heads 136 bytes apart
    ({11: 1 << 23}, fa.FA_ERR_UNSUPPORTED, "2^31"),     # o rows 2^24 bytes apart
    ({12: -4}, fa.FA_ERR_INVALID_ARG, "lse strides"),
])
def test_fwd_strided_validation(edit, status, msg):
    if edit == "null":
        st = "null"
    else:
        st = [2 * 16 * 4 * 64, 64, 4 * 64, 32 * 2 * 64, 64, 2 * 64, 32 * 2 * 64, 64, 2 * 64, 16 * 4 * 64, 64, 4 * 64,
              64, 16]
        for i, v in edit.items():
            st[i] = v
    assert _fwd_strided(st) == status
    assert msg in fa.last_error()


def test_bwd_strided_validation():
    L = fa.lib()
    B, H, Hkv, Nq, Nk, D = 1, 4, 2, 16, 32, 64
    ws = fa.bwd_workspace_size(B, H, Nq, D, fa.FA_BWD_DETERMINISTIC)
    q, k = _bnhd(B, H, Hkv, Nq, Nk, D)
    good = q + k + k + q + q + q + k + k + [H * Nq, Nq]

    def call(st, variant=fa.FA_BWD_DETERMINISTIC, wsb=ws):
        arr = None if st is None else (ctypes.c_longlong * 26)(*st)
        return L.fa_bwd_strided(P, P, P, P, P, P, P, P, P, B, H, Hkv, Nq, Nk, D, 1, -1, 0.1, fa.FA_BF16, variant, P,
                                wsb, arr, None)

    assert call(None) == fa.FA_ERR_INVALID_ARG and "NULL" in fa.last_error()
    assert call(good, variant=5) == fa.FA_ERR_INVALID_ARG and "variant" in fa.last_error()
    assert call(good, wsb=ws - 1) == fa.FA_ERR_WORKSPACE
    for i, name in ((14, "dO"), (17, "dq"), (20, "dk"), (23, "dv")):
        bad = list(good)
        bad[i] = D - 8  # row stride below D
        assert call(bad) == fa.FA_ERR_INVALID_ARG and name in fa.last_error(), name
    bad = list(good)
    bad[13] = 1 << 30  # dO heads 2^31 bytes apart: the 2 query heads of a group cannot share one 32-bit range
    assert call(bad) == fa.FA_ERR_UNSUPPORTED and "dO" in fa.last_error()


def test_varlen_validation():
    L = fa.lib()
    B, H, Hkv, D, Tq, Tk = 3, 4, 2, 64, 100, 150
    ws = fa.bwd_workspace_size(1, H, Tq, D, fa.FA_BWD_DETERMINISTIC)

    def f(cu_q=P, cu_k=P, Tq=Tq, Tk=Tk, mq=50, mk=60, D=D):
        return L.fa_fwd_varlen(P, P, P, P, P, cu_q, cu_k, B, H, Hkv, Tq, Tk, mq, mk, D, 1, -1, 0.125, fa.FA_BF16,
                               None)

    def b(wsb=ws, variant=fa.FA_BWD_DETERMINISTIC, cu_k=P):
        return L.fa_bwd_varlen(P, P, P, P, P, P, P, P, P, P, cu_k, B, H, Hkv, Tq, Tk, 50, 60, D, 1, -1, 0.125,
                               fa.FA_BF16, variant, P, wsb, None)

    assert f(cu_q=None) == fa.FA_ERR_INVALID_ARG and "cu_seqlens_q" in fa.last_error()
    assert f(cu_k=None) == fa.FA_ERR_INVALID_ARG and "cu_seqlens_k" in fa.last_error()
    assert f(cu_q=P + 2) == fa.FA_ERR_INVALID_ARG and "aligned" in fa.last_error()
    assert f(Tq=0) == fa.FA_ERR_INVALID_ARG and "total" in fa.last_error()
    assert f(mq=0) == fa.FA_ERR_INVALID_ARG
    assert f(D=80) == fa.FA_ERR_UNSUPPORTED
    assert b(wsb=ws - 1) == fa.FA_ERR_WORKSPACE
    assert b(variant=2) == fa.FA_ERR_INVALID_ARG
    assert b(cu_k=None) == fa.FA_ERR_INVALID_ARG


def test_block_sparse_validation():
    L = fa.lib()
    st = (ctypes.c_longlong * 3)(64, 16, 4)
    bad_st = (ctypes.c_longlong * 3)(64, -16, 4)

    def lists(mask=P, strides=st, B=1, H=2, Nq=500, Nk=500, causal=1, window=-1, ptrs=(P, P, P, P)):
        return L.fa_block_lists(mask, strides, B, H, Nq, Nk, causal, window, *ptrs, None)

    assert lists(mask=None) == fa.FA_ERR_INVALID_ARG and "mask" in fa.last_error()
    assert lists(strides=None) == fa.FA_ERR_INVALID_ARG and "mask_strides" in fa.last_error()
    assert lists(strides=bad_st) == fa.FA_ERR_INVALID_ARG and "strides" in fa.last_error()
    assert lists(Nq=0) == fa.FA_ERR_INVALID_ARG
    assert lists(causal=2) == fa.FA_ERR_INVALID_ARG
    assert lists(window=-3) == fa.FA_ERR_INVALID_ARG
    assert lists(ptrs=(P, None, P, P)) == fa.FA_ERR_INVALID_ARG and "block-list" in fa.last_error()
    assert lists(ptrs=(P, P, P + 2, P)) == fa.FA_ERR_INVALID_ARG and "aligned" in fa.last_error()

    def fwd(kvc=P, kvi=P, D=64):
        return L.fa_fwd_sparse(P, P, P, P, P, 1, 2, 2, 500, 500, D, 1, -1, 0.125, fa.FA_BF16, kvc, kvi, None)

    assert fwd(kvc=None) == fa.FA_ERR_INVALID_ARG
    assert fwd(kvi=P + 1) == fa.FA_ERR_INVALID_ARG
    assert fwd(D=96) == fa.FA_ERR_UNSUPPORTED
    ws = fa.bwd_workspace_size(1, 2, 500, 64, fa.FA_BWD_DETERMINISTIC)

    def bwd(variant=fa.FA_BWD_DETERMINISTIC, qi=P, wsb=ws):
        return L.fa_bwd_sparse(P, P, P, P, P, P, P, P, P, 1, 2, 2, 500, 500, 64, 1, -1, 0.125, fa.FA_BF16, variant,
                               P, P, P, qi, P, wsb, None)

    assert bwd(variant=2) == fa.FA_ERR_INVALID_ARG
    assert bwd(qi=None) == fa.FA_ERR_INVALID_ARG
    assert bwd(wsb=ws - 1) == fa.FA_ERR_WORKSPACE


def _bwd_noalloc(**kw):
    a = dict(B=1, H=1, N=16, D=64, causal=0, scale=0.125, dtype=fa.FA_BF16, variant=fa.FA_BWD_DETERMINISTIC)
    a.update(kw)
    return fa.lib().fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, a["B"], a["H"], a["N"], a["D"], a["causal"],
                                   a["scale"], a["dtype"], a["variant"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(N=0), fa.FA_ERR_INVALID_ARG, ">= 1"),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG, "scale"),
    (dict(variant=5), fa.FA_ERR_INVALID_ARG, "variant"),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED, "FA_BF16"),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED, "D=96"),
    # atomic variant at B4 H16 N2048 D128: 1 MiB of row statistics + 64 MiB of dQ accumulator > 64 MiB
    (dict(B=4, H=16, N=2048, D=128, variant=fa.FA_BWD_ATOMIC), fa.FA_ERR_WORKSPACE, "static scratch"),
    (dict(B=64, H=64, N=4096, D=64), fa.FA_ERR_WORKSPACE, "static scratch"),
])
def test_bwd_noalloc_validation(kw, status, msg):
    """fa_bwd_noalloc validates like fa_bwd and refuses problems beyond its static scratch, before any HIP call."""
    assert _bwd_noalloc(**kw) == status
    assert msg in fa.last_error()

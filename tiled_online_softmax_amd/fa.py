"""ctypes binding for libfa.so (argument marshalling only).

Every function here checks tensor placement/shape, allocates outputs with
torch (device memory is torch's job), and calls the matching C entry point of
include/fa.h on torch's current stream. All arithmetic runs in the HIP
kernels; there is no fallback: if libfa.so is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import functools
import math
import os
from typing import Optional, Tuple

import torch

# FA_LIBRARY selects another build of the library (e.g. the host-sanitised one, see build.py).
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_BF16, FA_FP8_E4M3 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, 1, 2, 3, 4
FA_BWD_ATOMIC, FA_BWD_DETERMINISTIC = 0, 1

EXPORTED = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_general", "fa_fwd_strided", "fa_fwd_varlen", "fa_block_lists",
            "fa_fwd_sparse", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_fp8_general", "fa_fwd_fp8_varlen", "fa_quantize_fp8",
            "fa_bwd_workspace_size", "fa_bwd",
            "fa_bwd_gqa", "fa_bwd_general", "fa_bwd_strided", "fa_bwd_sparse", "fa_bwd_varlen", "fa_bwd_dkdv",
            "fa_bwd_noalloc", "fa_status_string", "fa_last_error")
BLOCK = 128  # rows and columns of a block of a block-sparse mask


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by tiled_online_softmax_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m tiled_online_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.fa_fwd.argtypes = [_vp] * 5 + [_i] * 5 + [_f, _i, _vp]
        L.fa_fwd_gqa.argtypes = [_vp] * 5 + [_i] * 6 + [_f, _i, _vp]
        L.fa_fwd_general.argtypes = [_vp] * 5 + [_i] * 8 + [_f, _i, _vp]
        L.fa_fwd_strided.argtypes = [_vp] * 5 + [_i] * 8 + [_f, _i, _vp, _vp]
        L.fa_fwd_varlen.argtypes = [_vp] * 7 + [_i] * 10 + [_f, _i, _vp]
        L.fa_block_lists.argtypes = [_vp, _vp] + [_i] * 6 + [_vp] * 5
        L.fa_fwd_sparse.argtypes = [_vp] * 5 + [_i] * 8 + [_f, _i, _vp, _vp, _vp]
        L.fa_fwd_ex.argtypes = [_vp] * 5 + [_i] * 5 + [_f, _i, _f, _vp]
        L.fa_fwd_fp8.argtypes = [_vp] * 5 + [_i] * 5 + [_f] + [_vp] * 3 + [_vp]
        L.fa_fwd_fp8_general.argtypes = [_vp] * 5 + [_i] * 8 + [_f] + [_vp] * 3 + [_vp]
        L.fa_fwd_fp8_varlen.argtypes = [_vp] * 7 + [_i] * 10 + [_f] + [_vp] * 3 + [_vp]
        L.fa_quantize_fp8.argtypes = [_vp, _sz, _vp, _vp, _vp]
        L.fa_bwd_workspace_size.argtypes = [_i] * 6
        L.fa_bwd_workspace_size.restype = _sz
        L.fa_bwd.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i, _vp, _sz, _vp]
        L.fa_bwd_gqa.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _i, _i, _vp, _sz, _vp]
        L.fa_bwd_general.argtypes = [_vp] * 9 + [_i] * 8 + [_f, _i, _i, _vp, _sz, _vp]
        L.fa_bwd_strided.argtypes = [_vp] * 9 + [_i] * 8 + [_f, _i, _i, _vp, _sz, _vp, _vp]
        L.fa_bwd_varlen.argtypes = [_vp] * 11 + [_i] * 10 + [_f, _i, _i, _vp, _sz, _vp]
        L.fa_bwd_sparse.argtypes = [_vp] * 9 + [_i] * 8 + [_f, _i, _i] + [_vp] * 4 + [_vp, _sz, _vp]
        L.fa_bwd_dkdv.argtypes = [_vp] * 8 + [_i] * 5 + [_f, _i, _vp, _sz, _vp]
        L.fa_bwd_noalloc.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i, _vp]
        L.fa_status_string.argtypes = [_i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_last_error.argtypes = []
        L.fa_last_error.restype = ctypes.c_char_p
        for name in ("fa_fwd", "fa_fwd_gqa", "fa_fwd_general", "fa_fwd_strided", "fa_fwd_varlen", "fa_block_lists",
                     "fa_fwd_sparse", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_fp8_general", "fa_fwd_fp8_varlen",
                     "fa_quantize_fp8", "fa_bwd", "fa_bwd_gqa",
                     "fa_bwd_general", "fa_bwd_strided", "fa_bwd_sparse", "fa_bwd_varlen", "fa_bwd_dkdv",
                     "fa_bwd_noalloc"):
            getattr(L, name).restype = _i
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def last_error() -> str:
    return lib().fa_last_error().decode()


def _check(status: int):
    if status != FA_OK:
        raise FAError(status, last_error())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_qkv(*ts: torch.Tensor, kv=(), same_len=True, dense=True):
    """q-shaped tensors `ts` and K/V-shaped tensors `kv` (same B and D, H a multiple of their head count,
    and the same length unless `same_len` is False); contiguous, or with only D contiguous if not `dense`."""
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, N, D]")
    for t in tuple(ts) + tuple(kv):
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("tensors must share dtype and device")
        if dense and not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, D]")
        if not dense and t.stride(-1) != 1:
            raise ValueError("the head dimension D must be contiguous")
    for t in ts:
        if t.shape != ref.shape:
            raise ValueError("q-shaped tensors must share one shape")
    if kv:
        k0 = kv[0]
        for t in kv:
            if t.dim() != 4 or t.shape != k0.shape:
                raise ValueError("k and v must share one shape")
        B, H, N, D = ref.shape
        if k0.shape[0] != B or k0.shape[3] != D or k0.shape[1] < 1 or H % k0.shape[1]:
            raise ValueError("k/v must be [B, Hkv, Nk, D] with Hkv dividing the query heads")
        if same_len and k0.shape[2] != N:
            raise ValueError("k/v must have as many rows as q here")


def _strides(*ts: torch.Tensor, lse: torch.Tensor):
    """Host array of element strides: (batch, head, row) of each [B, H, N, D] tensor, then lse (batch, head)."""
    if lse.stride(2) != 1:
        raise ValueError("lse rows must be contiguous")
    vals = [x for t in ts for x in t.stride()[:3]] + list(lse.stride()[:2])
    return (ctypes.c_longlong * len(vals))(*vals)


def _dense(*ts) -> bool:
    return all(t is None or t.is_contiguous() for t in ts)


def _check_like(t: torch.Tensor, shape, dtype, device, name: str, contiguous: bool = True):
    """A caller-supplied tensor that a kernel reads or writes through a raw pointer: the C ABI sees only the
    pointer, so its shape, dtype and device must be exactly the expected ones (else a kernel would run past its
    end). `contiguous`: the whole tensor contiguous; otherwise its last dimension."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device} "
                         f"(got {t.dtype} {tuple(t.shape)} on {t.device})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have its last dimension contiguous")


def _workspace(workspace: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return workspace


def _on_device(fn):
    """Run a binding with the device of its first tensor argument current (the kernels launch on that
    device's current torch stream)."""

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        t = args[0] if args else None
        if isinstance(t, torch.Tensor) and t.is_cuda:
            with torch.cuda.device(t.device):
                return fn(*args, **kwargs)
        return fn(*args, **kwargs)

    return wrapper


@_on_device
def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
        rescale_log2: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, window: Optional[int] = None,
        block_lists: Optional["BlockLists"] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward. Returns (O, lse); O is float32 for float32 inputs, bf16 otherwise.

    k, v may have fewer heads (grouped-query) and a different length than q (causal is then
    aligned at the bottom right); `window` (>= 0) keeps only the keys from i + Nk - Nq - window on.
    Tensors may be any [B, H, N, D] views with D contiguous (e.g. x.view(B, N, H, D).transpose(1, 2));
    non-contiguous ones go through fa_fwd_strided. `block_lists` (from block_lists()) makes the call
    block-sparse (fa_fwd_sparse, contiguous tensors).
    """
    dense = _dense(q, k, v, out, lse)
    _check_qkv(q, kv=(k, v), same_len=False, dense=dense)
    B, H, N, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    odt = torch.float32 if code == FA_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_like(out, q.shape, odt, q.device, "out", contiguous=dense)
    _check_like(lse, (B, H, N), torch.float32, q.device, "lse", contiguous=dense)
    if block_lists is not None:
        if not dense or rescale_log2 is not None:
            raise ValueError("block-sparse calls take contiguous tensors and the default rescale threshold")
        bl = block_lists
        bl.check(B, H, N, Nk, causal, window, q.device)
        _check(lib().fa_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                   Hkv, N, Nk, D, int(causal), -1 if window is None else int(window), scale, code,
                                   bl.kv_count.data_ptr(), bl.kv_index.data_ptr(), _stream(q)))
        return out, lse
    if not dense:
        if rescale_log2 is not None:
            raise ValueError("rescale_log2 is only taken with contiguous tensors")
        _check(lib().fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                    Hkv, N, Nk, D, int(causal), -1 if window is None else int(window), scale, code,
                                    _strides(q, k, v, out, lse=lse), _stream(q)))
        return out, lse
    if Nk != N or window is not None:
        if rescale_log2 is not None:
            raise ValueError("rescale_log2 is only taken with equal lengths and no window")
        _check(lib().fa_fwd_general(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                    Hkv, N, Nk, D, int(causal), -1 if window is None else int(window), scale, code,
                                    _stream(q)))
        return out, lse
    if Hkv != H:
        if rescale_log2 is not None:
            raise ValueError("rescale_log2 is only taken with as many K/V heads as query heads")
        _check(lib().fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv,
                                N, D, int(causal), scale, code, _stream(q)))
        return out, lse
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, D, int(causal), scale,
            code)
    if rescale_log2 is None:
        _check(lib().fa_fwd(*args, _stream(q)))
    else:
        _check(lib().fa_fwd_ex(*args, float(rescale_log2), _stream(q)))
    return out, lse


@_on_device
def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
            q_descale: Optional[torch.Tensor] = None, k_descale: Optional[torch.Tensor] = None,
            v_descale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, window: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """FP8 (e4m3 codes, uint8 or float8_e4m3fn tensors) forward with per-tensor descales (1-element device tensors).

    k, v may have fewer heads (grouped-query) and another length than q (causal aligned at the bottom right), and
    `window` (>= 0) keeps only the keys from i + Nk - Nq - window on (fa_fwd_fp8_general); contiguous tensors.
    """
    _check_qkv(q, kv=(k, v), same_len=False)
    _check_fp8(q)
    B, H, N, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_like(out, q.shape, torch.bfloat16, q.device, "out")
    _check_like(lse, (B, H, N), torch.float32, q.device, "lse")
    d = [_descale_ptr(t, q) for t in (q_descale, k_descale, v_descale)]
    if Hkv == H and Nk == N and window is None:
        _check(lib().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, D,
                                int(causal), scale, *d, _stream(q)))
    else:
        _check(lib().fa_fwd_fp8_general(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                                        H, Hkv, N, Nk, D, int(causal), -1 if window is None else int(window), scale,
                                        *d, _stream(q)))
    return out, lse


def _check_fp8(q: torch.Tensor):
    if q.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError("the FP8 forward takes e4m3 codes (uint8 or float8_e4m3fn tensors)")


def _descale_ptr(t: Optional[torch.Tensor], q: torch.Tensor):
    if t is None:
        return None
    if t.dtype != torch.float32 or t.device != q.device or t.numel() < 1:
        raise ValueError("descales must be float32 tensors on q's device with one element")
    return t.data_ptr()


@_on_device
def fwd_fp8_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
                   scale: Optional[float] = None, window: Optional[int] = None, q_descale=None, k_descale=None,
                   v_descale=None, out=None, lse=None):
    """Packed variable-length FP8 forward (fa_fwd_fp8_varlen): e4m3 codes q [total_q, H, D], k, v [total_k, Hkv, D],
    per-tensor descales as in fwd_fp8. Returns (O bf16 [total_q, H, D], lse [H, total_q])."""
    _check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _check_fp8(q)
    Tq, H, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_like(out, q.shape, torch.bfloat16, q.device, "out")
    _check_like(lse, (H, Tq), torch.float32, q.device, "lse")
    d = [_descale_ptr(t, q) for t in (q_descale, k_descale, v_descale)]
    _check(lib().fa_fwd_fp8_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Hkv, Tq, Tk,
                                   int(max_seqlen_q), int(max_seqlen_k), D, int(causal),
                                   -1 if window is None else int(window), scale, *d, _stream(q)))
    return out, lse


@_on_device
def quantize_fp8(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-tensor e4m3 quantisation of a float32 device tensor: returns (codes uint8, descale float32[1])."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("quantize_fp8 takes a contiguous float32 device tensor")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    descale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().fa_quantize_fp8(x.data_ptr(), x.numel(), codes.data_ptr(), descale.data_ptr(), _stream(x)))
    return codes, descale


def bwd_workspace_size(B: int, H: int, N: int, D: int, variant: int = FA_BWD_DETERMINISTIC) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, N, D, FA_BF16, variant))


@_on_device
def bwd(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None, variant: int = FA_BWD_DETERMINISTIC,
        workspace: Optional[torch.Tensor] = None, dq=None, dk=None, dv=None, window: Optional[int] = None,
        block_lists: Optional["BlockLists"] = None):
    """Attention backward (bf16). Returns (dQ, dK, dV) as bf16 tensors; dK, dV have k's shape.

    The default variant is the atomics-free one: bitwise reproducible and, on MI355X, about twice as
    fast as FA_BWD_ATOMIC (which needs no second pass over the keys but adds dQ with float atomics).

    Non-contiguous [B, H, N, D] views (D contiguous) go through fa_bwd_strided."""
    dense = _dense(q, k, v, o, do, dq, dk, dv, lse)
    _check_qkv(q, o, do, kv=(k, v), same_len=False, dense=dense)
    B, H, N, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check_like(lse, (B, H, N), torch.float32, q.device, "lse", contiguous=dense)
    workspace = _workspace(workspace, bwd_workspace_size(B, H, N, D, variant), q.device)
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_like(t, like.shape, q.dtype, q.device, name, contiguous=dense)
    if block_lists is not None:
        if not dense:
            raise ValueError("block-sparse calls take contiguous tensors")
        bl = block_lists
        bl.check(B, H, N, Nk, causal, window, q.device)
        _check(lib().fa_bwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, Nk, D,
                                   int(causal), -1 if window is None else int(window), scale, _dtype_code(q),
                                   variant, bl.kv_count.data_ptr(), bl.kv_index.data_ptr(), bl.q_count.data_ptr(),
                                   bl.q_index.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(q)))
        return dq, dk, dv
    if not dense:
        _check(lib().fa_bwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, Nk, D,
                                    int(causal), -1 if window is None else int(window), scale, _dtype_code(q),
                                    variant, workspace.data_ptr(), workspace.numel(),
                                    _strides(q, k, v, o, do, dq, dk, dv, lse=lse), _stream(q)))
        return dq, dk, dv
    if Nk != N or window is not None:
        _check(lib().fa_bwd_general(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, Nk, D,
                                    int(causal), -1 if window is None else int(window), scale, _dtype_code(q),
                                    variant, workspace.data_ptr(), workspace.numel(), _stream(q)))
        return dq, dk, dv
    if Hkv != H:
        _check(lib().fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, D,
                                int(causal), scale, _dtype_code(q), variant, workspace.data_ptr(), workspace.numel(),
                                _stream(q)))
        return dq, dk, dv
    _check(lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, int(causal), scale, _dtype_code(q),
                        variant, workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dq, dk, dv


@_on_device
def bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
                variant: int = FA_BWD_DETERMINISTIC, dq=None, dk=None, dv=None):
    """Attention backward (bf16, contiguous [B, H, N, D]) through fa_bwd_noalloc: the library takes its
    workspace from a static device array (FA_NOALLOC_SCRATCH_BYTES), so the C call allocates nothing.
    Outputs the caller does not pass are allocated here by torch. Returns (dQ, dK, dV)."""
    _check_qkv(q, k, v, o, do)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check_like(lse, (B, H, N), torch.float32, q.device, "lse")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_like(t, q.shape, q.dtype, q.device, name)
    _check(lib().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, int(causal),
                                scale, _dtype_code(q), variant, _stream(q)))
    return dq, dk, dv


@_on_device
def bwd_dkdv(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
             workspace: Optional[torch.Tensor] = None, dk=None, dv=None):
    """dK and dV only (bf16), the key-tile pass of the backward. Returns (dK, dV)."""
    _check_qkv(q, k, v, o, do)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check_like(lse, (B, H, N), torch.float32, q.device, "lse")
    workspace = _workspace(workspace, bwd_workspace_size(B, H, N, D, FA_BWD_DETERMINISTIC), q.device)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_like(dk, k.shape, q.dtype, q.device, "dk")
    _check_like(dv, v.shape, q.dtype, q.device, "dv")
    _check(lib().fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             dk.data_ptr(), dv.data_ptr(), B, H, N, D, int(causal), scale, _dtype_code(q),
                             workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dk, dv


def _check_varlen(q, k, v, cu_q, cu_k):
    for t in (q, k, v):
        if t.dim() != 3 or not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("packed tensors must be contiguous [total, heads, D] tensors of one dtype on one device")
    if k.shape != v.shape or k.shape[2] != q.shape[2] or q.shape[1] % k.shape[1]:
        raise ValueError("k, v must be [total_k, Hkv, D] with Hkv dividing q's heads")
    for c in (cu_q, cu_k):
        if c.dtype != torch.int32 or c.device != q.device or not c.is_contiguous() or c.dim() != 1:
            raise ValueError("cu_seqlens must be contiguous int32 tensors on q's device")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 >= 2 entries")


@_on_device
def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
               scale: Optional[float] = None, window: Optional[int] = None, out=None, lse=None):
    """Packed variable-length forward: q [total_q, H, D], k, v [total_k, Hkv, D], int32 offsets [B + 1].
    Returns (O [total_q, H, D], lse [H, total_q])."""
    _check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k)
    Tq, H, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    odt = torch.float32 if code == FA_F32 else torch.bfloat16
    out = torch.empty(q.shape, dtype=odt, device=q.device) if out is None else out
    lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_like(out, q.shape, odt, q.device, "out")
    _check_like(lse, (H, Tq), torch.float32, q.device, "lse")
    _check(lib().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Hkv, Tq, Tk,
                               int(max_seqlen_q), int(max_seqlen_k), D, int(causal),
                               -1 if window is None else int(window), scale, code, _stream(q)))
    return out, lse


@_on_device
def bwd_varlen(q, k, v, o, do, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
               causal: bool = False, scale: Optional[float] = None, window: Optional[int] = None,
               variant: int = FA_BWD_DETERMINISTIC, workspace=None, dq=None, dk=None, dv=None):
    """Gradients of fwd_varlen (bf16). Returns (dQ, dK, dV) in the packed layouts (new dK, dV are zeroed
    first: key rows outside every sequence are not written)."""
    _check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k)
    Tq, H, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check_like(o, q.shape, q.dtype, q.device, "o")
    _check_like(do, q.shape, q.dtype, q.device, "do")
    _check_like(lse, (H, Tq), torch.float32, q.device, "lse")
    workspace = _workspace(workspace, bwd_workspace_size(1, H, Tq, D, variant), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.zeros_like(k) if dk is None else dk
    dv = torch.zeros_like(v) if dv is None else dv
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_like(t, like.shape, q.dtype, q.device, name)
    _check(lib().fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(),
                               cu_seqlens_k.data_ptr(), B, H, Hkv, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), D,
                               int(causal), -1 if window is None else int(window), scale, _dtype_code(q), variant,
                               workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dq, dk, dv


class BlockLists:
    """Device block lists of a block-sparse mask (fa_block_lists) and the geometry they were built for."""

    def __init__(self, kv_count, kv_index, q_count, q_index, geometry):
        self.kv_count, self.kv_index, self.q_count, self.q_index = kv_count, kv_index, q_count, q_index
        self.geometry = geometry

    def check(self, B, H, Nq, Nk, causal, window, device=None):
        if self.geometry != (B, H, Nq, Nk, bool(causal), -1 if window is None else int(window)):
            raise ValueError(f"block lists were built for {self.geometry}, not {(B, H, Nq, Nk, causal, window)}")
        if device is not None and self.kv_index.device != device:
            raise ValueError(f"block lists live on {self.kv_index.device}, the tensors on {device}")


@_on_device
def block_lists(mask: torch.Tensor, Nq: int, Nk: int, causal: bool = False, window: Optional[int] = None
                ) -> BlockLists:
    """Block lists of a [B, H, ceil(Nq / 128), ceil(Nk / 128)] mask (bool or uint8 device tensor, the last
    dimension contiguous; zero strides broadcast) for fwd(..., block_lists=) and bwd(..., block_lists=)."""
    if mask.dim() != 4 or not mask.is_cuda or mask.dtype not in (torch.bool, torch.uint8) or mask.stride(3) != 1:
        raise ValueError("mask must be a [B, H, nqb, nkb] bool/uint8 device tensor with the last dimension contiguous")
    B, H, nqb, nkb = mask.shape
    if nqb != -(-Nq // BLOCK) or nkb != -(-Nk // BLOCK):
        raise ValueError(f"mask must have ceil(Nq/{BLOCK}) x ceil(Nk/{BLOCK}) blocks")
    dev = mask.device
    kv_count = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    kv_index = torch.empty((B, H, nqb, nkb), dtype=torch.int32, device=dev)
    q_count = torch.empty((B, H, nkb), dtype=torch.int32, device=dev)
    q_index = torch.empty((B, H, nkb, nqb), dtype=torch.int32, device=dev)
    st = (ctypes.c_longlong * 3)(*[mask.stride(i) for i in range(3)])
    w = -1 if window is None else int(window)
    _check(lib().fa_block_lists(mask.data_ptr(), st, B, H, Nq, Nk, int(causal), w, kv_count.data_ptr(),
                                kv_index.data_ptr(), q_count.data_ptr(), q_index.data_ptr(), _stream(mask)))
    return BlockLists(kv_count, kv_index, q_count, q_index, (B, H, Nq, Nk, bool(causal), w))

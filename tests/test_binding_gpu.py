"""The Python binding refuses caller-supplied tensors that a kernel would read or write past.

The C ABI receives raw pointers only, so shapes, dtypes and devices of outputs, workspaces and auxiliary
inputs are checked in the binding. Every call here fails before any kernel is launched.
"""
import pytest
import torch

from tiled_online_softmax_amd import fa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def _t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def test_forward_outputs_checked():
    q, k, v = _t(1, 2, 64, 64), _t(1, 2, 64, 64), _t(1, 2, 64, 64)
    bad_out = [_t(1, 2, 63, 64), _t(1, 2, 64, 64, dtype=torch.float32), _t(2, 1, 64, 64)]
    for out in bad_out:
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, out=out)
    for lse in (_t(1, 2, 32, dtype=torch.float32), _t(1, 2, 64)):
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, lse=lse)
    # a non-contiguous but correctly shaped output goes through the strided entry point and is accepted
    wide = _t(1, 2, 64, 128)
    o, _ = fa.fwd(q, k, v, out=wide[..., :64])
    torch.cuda.synchronize()
    assert o.data_ptr() == wide.data_ptr()


def test_fp8_forward_outputs_checked():
    q = torch.zeros((1, 1, 64, 64), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        fa.fwd_fp8(q, q, q, out=_t(1, 1, 32, 64))
    with pytest.raises(ValueError):
        fa.fwd_fp8(q, q, q, q_descale=torch.ones(1, dtype=torch.float64, device=DEV))
    # bf16 (or any non-e4m3) tensors would be read as codes: refused
    for dt in (BF, torch.float32, torch.int8):
        x = _t(1, 1, 64, 64, dtype=dt)
        with pytest.raises(ValueError):
            fa.fwd_fp8(x, x, x)


def test_backward_outputs_and_workspace_checked():
    q, k, v, o, do = (_t(1, 2, 64, 64) for _ in range(5))
    lse = _t(1, 2, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, do, lse, dq=_t(1, 2, 32, 64))
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, do, lse, dk=_t(1, 2, 64, 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, do, _t(1, 2, 63, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, do, lse, workspace=torch.zeros(1 << 20, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        fa.bwd_dkdv(q, k, v, o, do, lse, dv=_t(1, 2, 64, 32))


def test_varlen_outputs_checked():
    q, k, v = _t(100, 2, 64), _t(100, 2, 64), _t(100, 2, 64)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        fa.fwd_varlen(q, k, v, cu, cu, 60, 60, out=_t(99, 2, 64))
    with pytest.raises(ValueError):
        fa.fwd_varlen(q, k, v, cu, cu, 60, 60, lse=_t(100, 2, dtype=torch.float32))
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, 60, 60)
    with pytest.raises(ValueError):
        fa.bwd_varlen(q, k, v, o[:50], o, lse, cu, cu, 60, 60)
    with pytest.raises(ValueError):
        fa.bwd_varlen(q, k, v, o, o, lse, cu, cu, 60, 60, dk=_t(100, 1, 64))
    torch.cuda.synchronize()

"""The Python binding refuses operands whose sizes or dtypes disagree before any
launch: the C ABI takes plain pointers and sizes, so a short mask or a narrower W
would otherwise be read past its end.  CPU only (the checks come first)."""

import pytest
import torch

from entropy_block_sparse_amd import flh_backward, flh_forward


def _ops(T=64, H=32, V=100, dt=torch.bfloat16):
    h = torch.zeros(T, H, dtype=dt)
    W = torch.zeros(V, H, dtype=dt)
    y = torch.zeros(T, dtype=torch.int64)
    f = torch.zeros(T, dtype=torch.float32)
    m = torch.ones(T, dtype=torch.uint8)
    return h, W, y, f, m


def test_forward_rejects_mismatched_operands():
    h, W, y, _, _ = _ops()
    with pytest.raises(ValueError, match="columns"):
        flh_forward(h, W[:, :16].contiguous(), y)
    with pytest.raises(ValueError, match="targets"):
        flh_forward(h, W, y[:10])
    with pytest.raises(TypeError, match="dtype"):
        flh_forward(h, W.float(), y)
    with pytest.raises(TypeError):
        flh_forward(h.half(), W.half(), y)
    with pytest.raises(ValueError, match="2-D"):
        flh_forward(h.reshape(-1), W, y)


@pytest.mark.parametrize("which", ["W_cols", "W_dtype", "targets", "lse", "entropy", "grad_logprob",
                                   "grad_entropy", "loss_mask"])
def test_backward_rejects_mismatched_operands(which):
    h, W, y, f, m = _ops()
    args = dict(h=h, W=W, targets=y, lse=f, entropy=f.clone(), grad_logprob=f.clone(),
                grad_entropy=f.clone(), loss_mask=m)
    if which == "W_cols":
        args["W"] = W[:, :24].contiguous()
    elif which == "W_dtype":
        args["W"] = W.float()
    else:
        args[which] = args[which][:-1]
    with pytest.raises((ValueError, TypeError)):
        flh_backward(**args)


def test_backward_rejects_metadata_of_another_length():
    h, W, y, f, m = _ops()

    class FakeMeta:
        T = 63

    with pytest.raises(ValueError, match="63"):
        flh_backward(h, W, y, f, f, f, f, m, FakeMeta())
    with pytest.raises(ValueError, match="loss mask"):
        flh_backward(h, W, y, f, f, f, f, None, FakeMeta())


def test_cpu_tensors_are_refused_after_the_checks():
    h, W, y, f, m = _ops()
    with pytest.raises(ValueError, match="HIP device"):
        flh_forward(h, W, y)
    with pytest.raises(ValueError, match="HIP device"):
        flh_backward(h, W, y, f, f, f, f, m, None)


def test_workspace_argument_is_checked_in_bytes():
    """A caller's workspace is measured in bytes (any dtype) and must be contiguous, on the
    call's device and large enough; too small or elsewhere raises instead of allocating."""
    from entropy_block_sparse_amd.ops import _use_workspace
    cpu = torch.device("cpu")
    ws, n = _use_workspace(torch.empty(100, dtype=torch.float32), 400, cpu)
    assert n == 400 and ws.numel() == 100
    with pytest.raises(ValueError, match="bytes"):
        _use_workspace(torch.empty(99, dtype=torch.float32), 400, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        _use_workspace(torch.empty(200, 4, dtype=torch.uint8).t(), 400, cpu)
    with pytest.raises(ValueError, match="device"):
        _use_workspace(torch.empty(400, dtype=torch.uint8), 400, torch.device("meta"))
    ws, n = _use_workspace(None, 1000, cpu)
    assert ws.dtype == torch.uint8 and n >= 1000

"""Host-side checks of the torch wrappers on tensors the caller passes in (out, lse, o, do,
workspace): a wrong shape, dtype, device or layout is a Python error before the library is
called, so the kernels never write past a buffer the caller made too small."""
import pytest
import torch

import exact_block_sparse_amd.api as api

CPU = torch.device("cpu")


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_tensor_arg_accepts_matching_tensors_in_any_layout():
    api._check_tensor_arg("out", bf(2, 3, 5, 64), (2, 3, 5, 64), CPU)
    bnhd = bf(2, 5, 3, 64).permute(0, 2, 1, 3)          # (B,N,H,d) memory as a [B,H,N,d] view
    api._check_tensor_arg("out", bnhd, (2, 3, 5, 64), CPU)


@pytest.mark.parametrize("bad,err", [
    (lambda: bf(2, 3, 4, 64), ValueError),                                    # too few rows
    (lambda: bf(2, 3, 5, 128), ValueError),                                   # other head dimension
    (lambda: torch.zeros(2, 3, 5, 64), TypeError),                            # fp32, not bf16
    (lambda: bf(2, 3, 64, 5).transpose(-1, -2), ValueError),                  # head dimension strided
    (lambda: "not a tensor", TypeError),
])
def test_tensor_arg_rejects(bad, err):
    with pytest.raises(err):
        api._check_tensor_arg("out", bad(), (2, 3, 5, 64), CPU)


def test_tensor_arg_rejects_another_device():
    with pytest.raises(ValueError):
        api._check_tensor_arg("out", bf(1, 1, 1, 64), (1, 1, 1, 64), torch.device("meta"))


@pytest.mark.parametrize("bad,err", [
    (lambda: torch.zeros(2, 3, 4), ValueError),                               # too small
    (lambda: torch.zeros(2, 3, 5, dtype=torch.float64), TypeError),
    (lambda: torch.zeros(2, 5, 3).transpose(1, 2), ValueError),               # not contiguous
    (lambda: torch.zeros(6, 5), ValueError),                                  # packed shape for fixed length
])
def test_stats_arg_rejects(bad, err):
    with pytest.raises(err):
        api._check_stats_arg("lse", bad(), (2, 3, 5), CPU)
    api._check_stats_arg("lse", torch.zeros(2, 3, 5), (2, 3, 5), CPU)


def test_workspace_is_counted_in_bytes():
    ws, n = api._workspace(torch.zeros(10, dtype=torch.float32), 16, CPU)
    assert n == 40
    ws, n = api._workspace(None, 300, CPU)
    assert n == 300 and ws.dtype == torch.uint8
    with pytest.raises(ValueError):
        api._workspace(torch.zeros(10, 2).t(), 16, CPU)

"""The binding's argument checks: every operand a plan or a run is handed is
checked against the problem before anything reaches the C library, so that a
wrongly sized, typed or placed tensor raises ValueError instead of letting a
kernel read or write past an allocation.  No GPU needed: a small stand-in
plays the device tensor (the checks only read its metadata)."""

import types

import numpy as np
import pytest
import torch

import window_spmm_amd as ws


class FakeDevTensor:
    """Metadata of a device tensor (shape, strides, dtype, device), no storage."""

    def __init__(self, shape, dtype=torch.int16, device=0, contiguous=True, is_cuda=True,
                 stride=None):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = types.SimpleNamespace(index=device)
        self.is_cuda = is_cuda
        self._contig = contiguous
        self._stride = stride or tuple(int(np.prod(self.shape[i + 1:])) for i in range(len(self.shape)))

    def data_ptr(self):
        return 4096

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def numel(self):
        return int(np.prod(self.shape)) if self.shape else 1

    def is_contiguous(self):
        return self._contig

    def dim(self):
        return len(self.shape)

    def stride(self, i=None):
        return self._stride if i is None else self._stride[i]


def _plan(fmt="bcsr", m=128, k=96, N=64, ab="bf16", ct="fp32", ws_bytes=0, col_major=0, dev=0):
    return ws.Plan(None, fmt, ws_bytes, (), {"m": m, "k": k, "N": N, "ab_dtype": ab, "c_dtype": ct,
                                             "col_major": col_major, "device": dev})


def _run_err(plan, B, C, workspace=None, match=None):
    with pytest.raises(ValueError, match=match):
        (ws.bcsr_run if plan.fmt == "bcsr" else ws.wcsr_run)(plan, B, C, workspace)


def test_run_rejects_wrong_shapes():
    p = _plan()
    good_b, good_c = FakeDevTensor((96, 64)), FakeDevTensor((128, 64), torch.float32)
    _run_err(p, FakeDevTensor((95, 64)), good_c, match="B has shape")
    _run_err(p, FakeDevTensor((96, 72)), good_c, match="B has shape")
    _run_err(p, good_b, FakeDevTensor((127, 64), torch.float32), match="C has shape")
    _run_err(p, good_b, FakeDevTensor((128, 56), torch.float32), match="C has shape")
    # a column-major plan takes B^T (N x k) and C^T (N x m)
    pc = _plan(col_major=1)
    _run_err(pc, good_b, FakeDevTensor((64, 128), torch.float32), match="column-major")
    _run_err(pc, FakeDevTensor((64, 96)), good_c, match="column-major")


def test_run_rejects_wrong_element_types():
    p = _plan(ct="fp32")
    good_b = FakeDevTensor((96, 64))
    # C of a fp32 plan must hold 4-byte floats, of a bf16 plan 16-bit codes
    _run_err(p, good_b, FakeDevTensor((128, 64), torch.bfloat16), match="C: torch dtype")
    _run_err(_plan(ct="bf16"), good_b, FakeDevTensor((128, 64), torch.float32), match="C: torch dtype")
    _run_err(_plan(ct="bf16"), good_b, FakeDevTensor((128, 64), torch.float16), match="C: torch dtype")
    # B of a 16-bit plan: 2-byte codes; of an FP8 plan: bytes
    _run_err(p, FakeDevTensor((96, 64), torch.float32), FakeDevTensor((128, 64), torch.float32),
             match="B: torch dtype")
    _run_err(_plan(ab="fp8"), FakeDevTensor((96, 64), torch.int16),
             FakeDevTensor((128, 64), torch.float32), match="B: torch dtype")


def test_run_rejects_host_and_foreign_device_tensors():
    p = _plan(dev=0)
    good_c = FakeDevTensor((128, 64), torch.float32)
    _run_err(p, FakeDevTensor((96, 64), is_cuda=False), good_c, match="device tensor")
    _run_err(p, FakeDevTensor((96, 64), device=1), good_c, match="cuda:1")
    _run_err(p, 1 << 20, good_c, match="must be a tensor")


def test_run_checks_the_workspace():
    p = _plan(fmt="wcsr", ab="fp16", ws_bytes=4096)
    B, C = FakeDevTensor((96, 64)), FakeDevTensor((128, 64), torch.float32)
    _run_err(p, B, C, None, match="needs a workspace")
    _run_err(p, B, C, FakeDevTensor((1023,), torch.float32), match="hold 4096 bytes")
    _run_err(p, B, C, FakeDevTensor((1024,), torch.float32, contiguous=False), match="hold 4096 bytes")
    _run_err(p, B, C, FakeDevTensor((1024,), torch.float32, device=2), match="plan's device")


def test_plan_checks_row_pointer_and_device_arrays():
    # BCSR 128 x 96, 64 x 32 blocks: ceil(128/64) + 1 = 3 row-pointer entries
    ptr = np.array([0, 2, 3], np.int32)
    idx = FakeDevTensor((3,), torch.int32)
    vals = FakeDevTensor((3 * 64 * 32,), torch.int16)
    with pytest.raises(ValueError, match="row pointer has 2 entries"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr[:2], idx, vals)
    with pytest.raises(ValueError, match="index array holds 2"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, FakeDevTensor((2,), torch.int32), vals)
    with pytest.raises(ValueError, match="value array holds"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, idx, FakeDevTensor((3 * 64 * 32 - 1,), torch.int16))
    with pytest.raises(ValueError, match="4-byte elements expected"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, FakeDevTensor((3,), torch.int16), vals)
    with pytest.raises(ValueError, match="2-byte elements expected"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, idx, FakeDevTensor((3 * 64 * 32,), torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, idx,
                     FakeDevTensor((3 * 64 * 32,), torch.int16, contiguous=False))
    with pytest.raises(ValueError, match="device tensor"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, idx, FakeDevTensor((3 * 64 * 32,), is_cuda=False))
    with pytest.raises(ValueError, match="cuda:1"):
        ws.bcsr_plan(128, 96, 64, 64, 32, ptr, idx, FakeDevTensor((3 * 64 * 32,), device=1))
    # WCSR: P packed columns need P indices and b_row * P values
    wptr = np.array([0, 16, 24], np.int32)
    with pytest.raises(ValueError, match="value array holds"):
        ws.wcsr_plan(32, 96, 64, 16, 8, wptr, FakeDevTensor((24,), torch.int32),
                     FakeDevTensor((16 * 24 - 8,), torch.int16))
    with pytest.raises(ValueError, match="row pointer has"):
        ws.wcsr_plan(33, 96, 64, 16, 8, wptr, FakeDevTensor((24,), torch.int32),
                     FakeDevTensor((16 * 24,), torch.int16))


def test_device_sparse_refuses_a_second_stream_on_its_own_workspace():
    """A plan with split windows writes partial tiles into its workspace: two
    streams sharing the object's single workspace would overwrite each other's
    partials, so a second stream must bring its own workspace."""
    obj = ws.DeviceSparse.__new__(ws.DeviceSparse)
    obj.fmt = "wcsr"
    obj.plan = _plan(fmt="wcsr", ab="fp16", ws_bytes=4096)
    obj.workspace = FakeDevTensor((1024,), torch.float32)
    obj._ws_stream = 111
    with pytest.raises(ValueError, match="another stream"):
        obj.run(FakeDevTensor((96, 64)), FakeDevTensor((128, 64), torch.float32), stream=222)

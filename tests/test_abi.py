"""The C-ABI library: it loads, exports every function include/window_spmm.h
declares, and its argument checks and error codes work without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import window_spmm_amd as ws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:spmm_status_t|const char \*|int64_t|void)\s*(spmm_\w+)\s*\(", text, re.M))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 14
    lib = ctypes.CDLL(ws.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert names == set(ws.EXPORTED)


def test_status_strings():
    for code in range(6):
        s = ws._lib.spmm_status_string(code).decode()
        assert s.startswith("SPMM_")
    assert ws._lib.spmm_status_string(99).decode() == "SPMM_ERR_UNKNOWN"


def _code(fn):
    with pytest.raises(ws.SpmmError) as e:
        fn()
    return e.value.code


def test_plan_argument_checks_before_device():
    ptr = np.array([0, 1], np.int32)
    # b_row not supported by any kernel
    assert _code(lambda: ws.bcsr_plan(8, 64, 64, 8, 8, ptr, 256, 256)) == ws.ERR_UNSUPPORTED
    # N not a multiple of 8
    assert _code(lambda: ws.bcsr_plan(16, 64, 60, 16, 16, ptr, 256, 256)) == ws.ERR_UNSUPPORTED
    # misaligned device arrays
    assert _code(lambda: ws.bcsr_plan(16, 64, 64, 16, 16, ptr, 258, 256)) == ws.ERR_UNSUPPORTED
    # k at the 24-bit limit of B row numbers
    assert _code(lambda: ws.wcsr_plan(16, 1 << 24, 64, 16, 8, np.array([0, 8], np.int32), 256, 256)) \
        == ws.ERR_UNSUPPORTED
    # row pointer going backwards
    assert _code(lambda: ws.bcsr_plan(32, 64, 64, 16, 16, np.array([0, 2, 1], np.int32), 256, 256)) \
        == ws.ERR_BAD_FORMAT
    # window width not a multiple of b_col
    assert _code(lambda: ws.wcsr_plan(16, 64, 64, 16, 8, np.array([0, 12], np.int32), 256, 256)) \
        == ws.ERR_BAD_FORMAT
    # split size not a multiple of 32
    assert _code(lambda: ws.wcsr_plan(16, 64, 64, 16, 8, np.array([0, 16], np.int32), 256, 256,
                                      split_cols=40)) == ws.ERR_INVALID_ARGUMENT


def test_run_with_null_plan_is_an_error():
    code = ws._lib.spmm_bcsr_run(None, None, 0, None, 0, None, None)
    assert code == ws.ERR_INVALID_ARGUMENT
    assert "null plan" in ws._lib.spmm_last_error().decode()
    assert ws._lib.spmm_plan_destroy(None) == ws.OK


def test_plan_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    ptr = np.array([0, 1], np.int32)
    assert _code(lambda: ws.bcsr_plan(16, 64, 64, 16, 16, ptr, 256, 256)) == ws.ERR_HIP


def test_launch_floor_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert ws._lib.spmm_launch_floor(None) == ws.ERR_HIP
    assert ws._lib.spmm_last_error().decode()


def test_recommended_ld():
    # pitches that are a multiple of 4 KiB get 2 KiB more from 16 KiB on, one
    # 128-byte line (64 elements, 128 for 1-byte data) below; others are kept
    assert ws.recommended_ld(65536, 2) == 66560
    assert ws.recommended_ld(65536, 4) == 66048
    assert ws.recommended_ld(65536, 1) == 67584
    assert ws.recommended_ld(8192, 2) == 9216
    assert ws.recommended_ld(16384, 1) == 18432
    assert ws.recommended_ld(4096, 2) == 4160
    assert ws.recommended_ld(4096, 1) == 4224
    assert ws.recommended_ld(1024, 4) == 1088
    assert ws.recommended_ld(2048, 2) == 2112
    assert ws.recommended_ld(16000, 2) == 16000
    assert ws.recommended_ld(128, 2) == 128
    assert ws.recommended_ld(1000, 2) == 1000
    assert ws.recommended_ld(1001, 2) == 1008
    assert ws.recommended_ld(0, 2) == 0


def test_plan_options_default_and_checks():
    """Option fields are range-checked before any device work (CPU-only
    check: these plans fail with INVALID_ARGUMENT, not a HIP error)."""
    o = ws.PlanOptions()
    ws._lib.spmm_plan_options_default(ctypes.byref(o))
    assert {n: getattr(o, n) for n, _ in o._fields_} == ws.PlanOptions.AUTO
    rp = np.array([0, 1], np.int32)
    bad = [{"kernel": 5}, {"kernel": -2}, {"cols_per_lane": 3}, {"waves_n": 3},
           {"waves_n": 4, "waves_k": 2}, {"distribution": 2}, {"order": -3},
           {"ranges_per_xcd": 65}, {"row_order": 5}]
    for opts in bad:
        with pytest.raises(ws.SpmmError, match="INVALID_ARGUMENT"):
            ws.bcsr_plan(64, 64, 64, 64, 64, rp, 16, 32, "bf16", "fp32", options=opts)
    # WCSR has only the generic kernel
    with pytest.raises(ws.SpmmError, match="INVALID_ARGUMENT"):
        ws.wcsr_plan(16, 64, 64, 16, 8, np.array([0, 8], np.int32), 16, 32, "fp16", "fp32",
                     options={"kernel": 1})
    with pytest.raises(ValueError):
        ws.PlanOptions.of({"tile": 3})


def test_allocation_failure_hook_gives_out_of_memory(monkeypatch):
    """SPMM_TEST_FAIL_ALLOC makes every guarded allocation fail: each builder,
    the split and the reordering calls then return OUT_OF_MEMORY with a
    message and write nothing; without it the same calls succeed."""
    import synth
    p = synth.random_problem(40, 50, 8, 0.1, seed=3)
    sq = synth.random_problem(40, 40, 8, 0.1, seed=4)  # square, for the reordering calls
    calls = {
        "bcsr": lambda: ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 16, 16),
        "bcsr8": lambda: ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals & 0x7F, 16, 16,
                                        code_bytes=1),
        "wcsr": lambda: ws.csr_to_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 16, 8),
        "split": lambda: ws.wcsr_split(np.array([0, 64, 64, 200], np.int32), 32),
        "rcm": lambda: ws.rcm_order(40, sq.row_ptr, sq.col_idx),
        "permute": lambda: ws.csr_permute(40, sq.row_ptr, sq.col_idx, sq.vals,
                                          np.arange(40, dtype=np.int32)),
    }
    for name, fn in calls.items():
        fn()  # succeeds without the hook
    monkeypatch.setenv("SPMM_TEST_FAIL_ALLOC", "1")
    for name, fn in calls.items():
        with pytest.raises(ws.SpmmError) as e:
            fn()
        assert e.value.code == ws.ERR_OUT_OF_MEMORY, name
        assert "allocation" in str(e.value), name
    monkeypatch.setenv("SPMM_TEST_FAIL_ALLOC", "0")
    for fn in calls.values():
        fn()


def test_tuned_plan_argument_checks_without_gpu():
    """The tuned plans check their own arguments before any device work: a null
    plan pointer or reps outside [0, 10000] is INVALID_ARGUMENT; without a GPU
    the automatic plan fails with a HIP error."""
    import torch
    ptr = np.array([0, 1], np.int32)
    sz = ctypes.c_size_t(0)
    h = ctypes.c_void_p(0)
    opt = ws.PlanOptions.of(None)
    args = (16, 64, 64, 16, 16, ptr.ctypes.data, 256, 256, 0, 2, ctypes.byref(opt), 512, 64, 1024, 64,
            None)
    assert ws._lib.spmm_bcsr_plan_tuned(None, *args, 0, None, ctypes.byref(sz)) == ws.ERR_INVALID_ARGUMENT
    assert ws._lib.spmm_bcsr_plan_tuned(ctypes.byref(h), *args, -1, None, ctypes.byref(sz)) \
        == ws.ERR_INVALID_ARGUMENT
    assert "reps" in ws._lib.spmm_last_error().decode()
    wptr = np.array([0, 8], np.int32)
    wargs = (16, 64, 64, 16, 8, wptr.ctypes.data, 256, 256, 0, 2, 0, ctypes.byref(opt), 512, 64,
             1024, 64, None)
    assert ws._lib.spmm_wcsr_plan_tuned(ctypes.byref(h), *wargs, 20000, None, ctypes.byref(sz)) \
        == ws.ERR_INVALID_ARGUMENT
    if not torch.cuda.is_available():
        assert ws._lib.spmm_bcsr_plan_tuned(ctypes.byref(h), *args, 0, None, ctypes.byref(sz)) == ws.ERR_HIP
        assert not h.value

"""Python binding of libwindow_spmm (BCSR / WCSR SpMM for MI355X, gfx950).

Argument marshalling only: every step of the SpMM runs in the native library
(host-side format builders in C++, the product in HIP kernels).  Device
buffers are torch tensors (or raw integer device addresses); torch provides
memory and streams, nothing else.  There is no fallback: if the native
library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwindow_spmm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("window_spmm_amd: native library %s is missing; build it with "
                      "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)

# torch is loaded first on purpose: it ships its own HIP runtime with the same
# soname as the system one, and the library must bind to the runtime that owns
# the tensors and streams it is handed.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARGUMENT, ERR_BAD_FORMAT, ERR_UNSUPPORTED, ERR_OUT_OF_MEMORY, ERR_HIP = range(6)
DTYPES = {"fp16": 0, "bf16": 1, "fp32": 2, "fp8": 3}
EXPORTED = [
    "spmm_csr_to_bcsr_count", "spmm_csr_to_bcsr", "spmm_csr_to_bcsr8", "spmm_csr_to_wcsr_count",
    "spmm_csr_to_wcsr",
    "spmm_wcsr_split_count", "spmm_wcsr_split", "spmm_bcsr_plan", "spmm_wcsr_plan",
    "spmm_bcsr_run", "spmm_wcsr_run", "spmm_plan_info", "spmm_plan_destroy",
    "spmm_status_string", "spmm_last_error", "spmm_recommended_ld", "spmm_rcm_order",
    "spmm_csr_permute", "spmm_plan_options_default", "spmm_bcsr_plan_ex", "spmm_wcsr_plan_ex",
    "spmm_launch_floor", "spmm_wcsr_run_noalloc", "spmm_bcsr_plan_tuned", "spmm_wcsr_plan_tuned",
]
# bytes of the library's static partial-tile scratch (SPMM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


class PlanInfo(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("tile_cols", ctypes.c_int32), ("waves_n", ctypes.c_int32),
                ("waves_k", ctypes.c_int32), ("cols_per_lane", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("ranges_per_xcd", ctypes.c_int32),
                ("col_major", ctypes.c_int32), ("tuned", ctypes.c_int32),
                ("split_cols", ctypes.c_int64), ("n_tasks", ctypes.c_int64),
                ("n_merges", ctypes.c_int64), ("n_slots", ctypes.c_int64),
                ("stored_entries", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class PlanOptions(ctypes.Structure):
    """spmm_plan_options_t: -1 / 0 = let the plan choose (see the C header)."""
    _fields_ = [("kernel", ctypes.c_int32), ("cols_per_lane", ctypes.c_int32),
                ("waves_n", ctypes.c_int32), ("waves_k", ctypes.c_int32),
                ("distribution", ctypes.c_int32), ("row_order", ctypes.c_int32),
                ("order", ctypes.c_int32), ("ranges_per_xcd", ctypes.c_int32),
                ("col_major", ctypes.c_int32)]

    AUTO = {"kernel": -1, "cols_per_lane": 0, "waves_n": 0, "waves_k": 0, "distribution": -1,
            "row_order": -1, "order": -1, "ranges_per_xcd": 0, "col_major": 0}

    @classmethod
    def of(cls, options=None):
        """From a dict of the fields to pin (others automatic), or None."""
        o = cls(**cls.AUTO)
        for name, value in (options or {}).items():
            if name not in cls.AUTO:
                raise ValueError("unknown plan option %r" % name)
            setattr(o, name, int(value))
        return o


_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_P64 = ctypes.POINTER(ctypes.c_int64)
_Psz = ctypes.POINTER(ctypes.c_size_t)
_sigs = {
    "spmm_csr_to_bcsr_count": [_i64, _i64, _vp, _vp, _i32, _i32, _P64],
    "spmm_csr_to_bcsr": [_i64, _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp],
    "spmm_csr_to_bcsr8": [_i64, _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp],
    "spmm_csr_to_wcsr_count": [_i64, _i64, _vp, _vp, _i32, _i32, _P64],
    "spmm_csr_to_wcsr": [_i64, _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp],
    "spmm_wcsr_split_count": [_i64, _vp, _i64, _P64, _P64],
    "spmm_wcsr_split": [_i64, _vp, _i64, _vp, _vp],
    "spmm_rcm_order": [_i64, _vp, _vp, _vp],
    "spmm_csr_permute": [_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "spmm_bcsr_plan": [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                       ctypes.c_int, ctypes.c_int, _Psz],
    "spmm_wcsr_plan": [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                       ctypes.c_int, ctypes.c_int, _i64, _Psz],
    "spmm_bcsr_plan_ex": [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                          ctypes.c_int, ctypes.c_int, ctypes.POINTER(PlanOptions), _Psz],
    "spmm_wcsr_plan_ex": [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                          ctypes.c_int, ctypes.c_int, _i64, ctypes.POINTER(PlanOptions), _Psz],
    "spmm_bcsr_plan_tuned": [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                             ctypes.c_int, ctypes.c_int, ctypes.POINTER(PlanOptions), _vp, _i64,
                             _vp, _i64, _vp, _i32, ctypes.POINTER(PlanOptions), _Psz],
    "spmm_wcsr_plan_tuned": [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                             ctypes.c_int, ctypes.c_int, _i64, ctypes.POINTER(PlanOptions), _vp,
                             _i64, _vp, _i64, _vp, _i32, ctypes.POINTER(PlanOptions), _Psz],
    "spmm_bcsr_run": [_vp, _vp, _i64, _vp, _i64, _vp, _vp],
    "spmm_wcsr_run": [_vp, _vp, _i64, _vp, _i64, _vp, _vp],
    "spmm_wcsr_run_noalloc": [_vp, _vp, _i64, _vp, _i64, _vp],
    "spmm_plan_info": [_vp, ctypes.POINTER(PlanInfo)],
    "spmm_plan_destroy": [_vp],
    "spmm_launch_floor": [_vp],
}
for _name, _args in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.spmm_status_string.argtypes = [ctypes.c_int]
_lib.spmm_status_string.restype = ctypes.c_char_p
_lib.spmm_last_error.argtypes = []
_lib.spmm_last_error.restype = ctypes.c_char_p
_lib.spmm_recommended_ld.argtypes = [ctypes.c_int64, ctypes.c_int32]
_lib.spmm_recommended_ld.restype = ctypes.c_int64
_lib.spmm_plan_options_default.argtypes = [ctypes.POINTER(PlanOptions)]
_lib.spmm_plan_options_default.restype = None


def recommended_ld(N: int, elem_bytes: int) -> int:
    """Leading dimension to allocate for an N-column operand (see the C header)."""
    return int(_lib.spmm_recommended_ld(int(N), int(elem_bytes)))


class SpmmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        name = _lib.spmm_status_string(code).decode()
        msg = _lib.spmm_last_error().decode()
        super().__init__("%s: %s (%s)" % (where, name, msg))


def _check(code: int, where: str):
    if code != OK:
        raise SpmmError(code, where)


def _host(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _codes8(a) -> np.ndarray:
    """8-bit codes from any integer array holding values 0..255 (e.g. FP8 codes
    kept in uint16 arrays); anything else is an error, never a truncation."""
    a = np.asarray(a)
    if a.dtype != np.uint8 and a.size and (int(a.min()) < 0 or int(a.max()) > 255):
        raise ValueError("8-bit codes must lie in 0..255")
    return np.ascontiguousarray(a, dtype=np.uint8)


def _hp(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)


def _dp(x) -> ctypes.c_void_p:
    """Device address of a torch tensor (or an integer address, or None)."""
    if x is None:
        return ctypes.c_void_p(0)
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    return ctypes.c_void_p(x.data_ptr())


# --------------------------------------------------------------------------
# host-side builders
# --------------------------------------------------------------------------

def csr_to_bcsr(m: int, k: int, row_ptr, col_idx, values, b_row: int, b_col: int,
                code_bytes: int = 2):
    """CSR -> BCSR ``(block_row_ptr, block_col_idx, blocks)`` (numpy).  Values
    are 16-bit codes, or 8-bit codes (FP8 E4M3) with ``code_bytes=1``."""
    if code_bytes not in (1, 2):
        raise ValueError("code_bytes must be 1 or 2")
    ct = np.uint8 if code_bytes == 1 else np.uint16
    rp, ci = _host(row_ptr, np.int32), _host(col_idx, np.int32)
    v = _codes8(values) if code_bytes == 1 else _host(values, ct)
    n = ctypes.c_int64(0)
    _check(_lib.spmm_csr_to_bcsr_count(m, k, _hp(rp), _hp(ci), b_row, b_col, ctypes.byref(n)),
           "spmm_csr_to_bcsr_count")
    brp = np.empty(-(-m // b_row) + 1, np.int32)
    bci = np.empty(n.value, np.int32)
    blk = np.empty(n.value * b_row * b_col, ct)
    fn, name = (_lib.spmm_csr_to_bcsr8, "spmm_csr_to_bcsr8") if code_bytes == 1 else \
        (_lib.spmm_csr_to_bcsr, "spmm_csr_to_bcsr")
    _check(fn(m, k, _hp(rp), _hp(ci), _hp(v), b_row, b_col, _hp(brp), _hp(bci), _hp(blk)), name)
    return brp, bci, blk


def csr_to_wcsr(m: int, k: int, row_ptr, col_idx, values, b_row: int, b_col: int):
    """CSR -> WCSR ``(window_row_ptr, window_col_idx, values)`` (numpy)."""
    rp, ci, v = _host(row_ptr, np.int32), _host(col_idx, np.int32), _host(values, np.uint16)
    P = ctypes.c_int64(0)
    _check(_lib.spmm_csr_to_wcsr_count(m, k, _hp(rp), _hp(ci), b_row, b_col, ctypes.byref(P)),
           "spmm_csr_to_wcsr_count")
    wrp = np.empty(-(-m // b_row) + 1, np.int32)
    wci = np.empty(P.value, np.int32)
    wv = np.empty(P.value * b_row, np.uint16)
    _check(_lib.spmm_csr_to_wcsr(m, k, _hp(rp), _hp(ci), _hp(v), b_row, b_col, _hp(wrp), _hp(wci),
                                 _hp(wv)), "spmm_csr_to_wcsr")
    return wrp, wci, wv


def wcsr_split(window_row_ptr, split_cols: int):
    """Task list ``(tasks int32[n,4], merges int32[s,3])`` for sub-task size T."""
    wrp = _host(window_row_ptr, np.int32)
    nw = wrp.size - 1
    nt, nm = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.spmm_wcsr_split_count(nw, _hp(wrp), split_cols, ctypes.byref(nt), ctypes.byref(nm)),
           "spmm_wcsr_split_count")
    tasks = np.empty((nt.value, 4), np.int32)
    merges = np.empty((nm.value, 3), np.int32)
    _check(_lib.spmm_wcsr_split(nw, _hp(wrp), split_cols, _hp(tasks), _hp(merges)), "spmm_wcsr_split")
    return tasks, merges


def rcm_order(n: int, row_ptr, col_idx) -> np.ndarray:
    """Reverse Cuthill-McKee order of a square CSR pattern: ``perm`` (int32[n]),
    new position i holds old vertex perm[i] (rules in the C header)."""
    rp, ci = _host(row_ptr, np.int32), _host(col_idx, np.int32)
    perm = np.empty(n, np.int32)
    _check(_lib.spmm_rcm_order(n, _hp(rp), _hp(ci), _hp(perm)), "spmm_rcm_order")
    return perm


def csr_permute(n: int, row_ptr, col_idx, values, perm):
    """Symmetric permutation P A P^T of a square CSR matrix:
    ``(row_ptr, col_idx, values)`` with entry (perm[i], perm[j]) moved to (i, j)."""
    rp, ci = _host(row_ptr, np.int32), _host(col_idx, np.int32)
    v, pm = _host(values, np.uint16), _host(perm, np.int32)
    orp = np.empty(n + 1, np.int32)
    oci = np.empty(ci.size, np.int32)
    ov = np.empty(ci.size, np.uint16)
    _check(_lib.spmm_csr_permute(n, _hp(rp), _hp(ci), _hp(v), _hp(pm), _hp(orp), _hp(oci), _hp(ov)),
           "spmm_csr_permute")
    return orp, oci, ov


# --------------------------------------------------------------------------
# plans and runs
# --------------------------------------------------------------------------

class Plan:
    """Owns a spmm_plan_t; keeps the device arrays it refers to alive and
    remembers the problem it was made for, so that runs can check their
    operands against it before anything reaches a kernel."""

    def __init__(self, handle, fmt: str, workspace_bytes: int, keep=(), problem=None):
        self._h = handle
        self.fmt = fmt
        self.workspace_bytes = int(workspace_bytes)
        self._keep = keep
        # m, k, N, ab_dtype, c_dtype, col_major, device index (None: unknown)
        self.problem = problem or {}

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def info(self) -> dict:
        pi = PlanInfo()
        _check(_lib.spmm_plan_info(self.handle, ctypes.byref(pi)), "spmm_plan_info")
        return pi.as_dict()

    def destroy(self):
        if self._h is not None:
            _lib.spmm_plan_destroy(self._h)
            self._h = None
            self._keep = ()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# Bytes per element of each dtype name, and the torch dtypes a tensor holding
# such elements may have (16-bit codes may also travel as raw int16/uint16).
_ELEM_BYTES = {"fp16": 2, "bf16": 2, "fp32": 4, "fp8": 1}
_TORCH_OK = {"fp32": ("float32",), "bf16": ("bfloat16", "int16", "uint16"),
             "fp16": ("float16", "int16", "uint16"), "fp8": ("uint8", "int8", "float8_e4m3fn")}


def _is_tensor(x) -> bool:
    return x is not None and not isinstance(x, int) and hasattr(x, "data_ptr")


def _check_dtype(name: str, t, dtype: str):
    tn = str(t.dtype).replace("torch.", "")
    if tn not in _TORCH_OK[dtype]:
        raise ValueError("%s: torch dtype %s does not hold %s elements (expected one of %s)"
                         % (name, tn, dtype, ", ".join(_TORCH_OK[dtype])))


def _check_device_array(name: str, t, elem_bytes: int, need: int, device=None):
    """A plan's device array: contiguous, on a GPU, elements of the right size,
    at least `need` of them.  Raw integer addresses are the caller's business."""
    if not _is_tensor(t):
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and t.device.index != device:
        raise ValueError("%s is on cuda:%s, the plan's other arrays on cuda:%s"
                         % (name, t.device.index, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.element_size() != elem_bytes:
        raise ValueError("%s holds %d-byte elements, %d-byte elements expected"
                         % (name, t.element_size(), elem_bytes))
    if t.numel() < need:
        raise ValueError("%s holds %d elements, the row pointer needs %d" % (name, t.numel(), need))


def _plan_checks(fmt, m, k, N, b_row, b_col, rp, d_idx, d_vals, ab_dtype, c_dtype, options):
    """Host-side checks of a plan call that the C library cannot make (it sees
    raw pointers): the row pointer's length and the device arrays' sizes.
    Returns the problem record the plan keeps for its runs."""
    if ab_dtype not in _ELEM_BYTES or c_dtype not in _ELEM_BYTES:
        raise ValueError("unknown dtype %r / %r" % (ab_dtype, c_dtype))
    if min(int(m), int(k), int(N)) < 0 or int(b_row) < 1 or int(b_col) < 1:
        raise ValueError("negative size or non-positive block size")
    nrow = -(-int(m) // int(b_row))
    if rp.ndim != 1 or rp.size != nrow + 1:
        raise ValueError("row pointer has %d entries, ceil(m / b_row) + 1 = %d expected"
                         % (rp.size, nrow + 1))
    total = int(rp[-1])
    if total < 0:
        raise ValueError("row pointer ends below 0")
    n_vals = total * int(b_row) * (int(b_col) if fmt == "bcsr" else 1)
    dev = d_idx.device.index if _is_tensor(d_idx) and d_idx.is_cuda else None
    _check_device_array("index array", d_idx, 4, total, dev)
    _check_device_array("value array", d_vals, _ELEM_BYTES[ab_dtype], n_vals, dev)
    if dev is None and _is_tensor(d_vals) and d_vals.is_cuda:
        dev = d_vals.device.index
    return {"m": int(m), "k": int(k), "N": int(N), "ab_dtype": ab_dtype, "c_dtype": c_dtype,
            "col_major": int((options or {}).get("col_major", 0)), "device": dev}


def bcsr_plan(m, k, N, b_row, b_col, h_block_row_ptr, d_block_col_idx, d_blocks,
              ab_dtype="bf16", c_dtype="fp32", options=None) -> Plan:
    """spmm_bcsr_plan_ex; ``options``: dict of PlanOptions fields to pin.
    ValueError if the row pointer's length or a device array's size, element
    size or device does not fit the problem."""
    rp = _host(h_block_row_ptr, np.int32)
    prob = _plan_checks("bcsr", m, k, N, b_row, b_col, rp, d_block_col_idx, d_blocks, ab_dtype,
                        c_dtype, options)
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    opt = PlanOptions.of(options)
    _check(_lib.spmm_bcsr_plan_ex(ctypes.byref(h), m, k, N, b_row, b_col, _hp(rp),
                                  _dp(d_block_col_idx), _dp(d_blocks), DTYPES[ab_dtype],
                                  DTYPES[c_dtype], ctypes.byref(opt), ctypes.byref(ws)),
           "spmm_bcsr_plan_ex")
    return Plan(h, "bcsr", ws.value, (d_block_col_idx, d_blocks), prob)


def wcsr_plan(m, k, N, b_row, b_col, h_window_row_ptr, d_window_col_idx, d_values,
              ab_dtype="fp16", c_dtype="fp32", split_cols=0, options=None) -> Plan:
    """spmm_wcsr_plan_ex; ``options``: dict of PlanOptions fields to pin.
    ValueError as for bcsr_plan."""
    rp = _host(h_window_row_ptr, np.int32)
    prob = _plan_checks("wcsr", m, k, N, b_row, b_col, rp, d_window_col_idx, d_values, ab_dtype,
                        c_dtype, options)
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    opt = PlanOptions.of(options)
    _check(_lib.spmm_wcsr_plan_ex(ctypes.byref(h), m, k, N, b_row, b_col, _hp(rp),
                                  _dp(d_window_col_idx), _dp(d_values), DTYPES[ab_dtype],
                                  DTYPES[c_dtype], int(split_cols), ctypes.byref(opt),
                                  ctypes.byref(ws)), "spmm_wcsr_plan_ex")
    return Plan(h, "wcsr", ws.value, (d_window_col_idx, d_values), prob)


def _options_dict(o: PlanOptions) -> dict:
    """The fields of `o` that are not automatic."""
    return {name: getattr(o, name) for name, auto in PlanOptions.AUTO.items()
            if getattr(o, name) != auto}


def bcsr_plan_tuned(m, k, N, b_row, b_col, h_block_row_ptr, d_block_col_idx, d_blocks, B, C,
                    ab_dtype="bf16", c_dtype="fp32", options=None, stream=None, reps=0):
    """spmm_bcsr_plan_tuned: times the candidate configurations on B and C
    (C is overwritten) and returns (plan, options it was made with)."""
    rp = _host(h_block_row_ptr, np.int32)
    prob = _plan_checks("bcsr", m, k, N, b_row, b_col, rp, d_block_col_idx, d_blocks, ab_dtype,
                        c_dtype, options)
    _run_checks(Plan(None, "bcsr", 0, (), prob), B, C, None, check_workspace=False)
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    opt, chosen = PlanOptions.of(options), PlanOptions.of(None)
    _check(_lib.spmm_bcsr_plan_tuned(ctypes.byref(h), m, k, N, b_row, b_col, _hp(rp),
                                     _dp(d_block_col_idx), _dp(d_blocks), DTYPES[ab_dtype],
                                     DTYPES[c_dtype], ctypes.byref(opt), _dp(B), _ld(B), _dp(C),
                                     _ld(C), _stream_handle(stream), int(reps),
                                     ctypes.byref(chosen), ctypes.byref(ws)),
           "spmm_bcsr_plan_tuned")
    return Plan(h, "bcsr", ws.value, (d_block_col_idx, d_blocks), prob), _options_dict(chosen)


def wcsr_plan_tuned(m, k, N, b_row, b_col, h_window_row_ptr, d_window_col_idx, d_values, B, C,
                    ab_dtype="fp16", c_dtype="fp32", split_cols=0, options=None, stream=None,
                    reps=0):
    """spmm_wcsr_plan_tuned: as bcsr_plan_tuned for WCSR (split_cols = 0 also
    times sub-task sizes)."""
    rp = _host(h_window_row_ptr, np.int32)
    prob = _plan_checks("wcsr", m, k, N, b_row, b_col, rp, d_window_col_idx, d_values, ab_dtype,
                        c_dtype, options)
    _run_checks(Plan(None, "wcsr", 0, (), prob), B, C, None, check_workspace=False)
    h = ctypes.c_void_p(0)
    ws = ctypes.c_size_t(0)
    opt, chosen = PlanOptions.of(options), PlanOptions.of(None)
    _check(_lib.spmm_wcsr_plan_tuned(ctypes.byref(h), m, k, N, b_row, b_col, _hp(rp),
                                     _dp(d_window_col_idx), _dp(d_values), DTYPES[ab_dtype],
                                     DTYPES[c_dtype], int(split_cols), ctypes.byref(opt), _dp(B),
                                     _ld(B), _dp(C), _ld(C), _stream_handle(stream), int(reps),
                                     ctypes.byref(chosen), ctypes.byref(ws)),
           "spmm_wcsr_plan_tuned")
    return Plan(h, "wcsr", ws.value, (d_window_col_idx, d_values), prob), _options_dict(chosen)


def _stream_handle(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def launch_floor(stream=None):
    """Enqueues one empty kernel on `stream` (spmm_launch_floor)."""
    _check(_lib.spmm_launch_floor(_stream_handle(stream)), "spmm_launch_floor")


def _ld(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        raise ValueError("B and C must be tensors (their leading dimension is read from them)")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("B and C must be 2-D with unit column stride")
    return int(t.stride(0))


def _run_checks(plan: Plan, B, C, workspace, check_workspace: bool = True):
    """Checks B, C and the workspace against the problem the plan was made for:
    shapes (k x N and m x N, or N x k and N x m for a column-major plan),
    element types, device, and the workspace size.  Raises ValueError; nothing
    is launched."""
    pr = plan.problem
    if not pr:
        return
    cm = pr["col_major"]
    want_b = (pr["N"], pr["k"]) if cm else (pr["k"], pr["N"])
    want_c = (pr["N"], pr["m"]) if cm else (pr["m"], pr["N"])
    for name, t, want, dt in (("B", B, want_b, pr["ab_dtype"]), ("C", C, want_c, pr["c_dtype"])):
        if t is None:
            continue
        if not _is_tensor(t):
            raise ValueError("%s must be a tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if pr["device"] is not None and t.device.index != pr["device"]:
            raise ValueError("%s is on cuda:%s, the plan on cuda:%s" % (name, t.device.index,
                                                                        pr["device"]))
        if tuple(t.shape) != want:
            raise ValueError("%s has shape %s, the plan needs %s%s" % (
                name, tuple(t.shape), want, " (column-major plan)" if cm else ""))
        _check_dtype(name, t, dt)
    if check_workspace and plan.workspace_bytes > 0:
        if not _is_tensor(workspace):
            raise ValueError("the plan needs a workspace tensor of %d bytes" % plan.workspace_bytes)
        if not workspace.is_cuda or (pr["device"] is not None and
                                     workspace.device.index != pr["device"]):
            raise ValueError("the workspace must be on the plan's device")
        if not workspace.is_contiguous() or \
                workspace.numel() * workspace.element_size() < plan.workspace_bytes:
            raise ValueError("the workspace must be contiguous and hold %d bytes"
                             % plan.workspace_bytes)


def bcsr_run(plan: Plan, B, C, workspace=None, stream=None):
    _run_checks(plan, B, C, workspace)
    _check(_lib.spmm_bcsr_run(plan.handle, _dp(B), _ld(B), _dp(C), _ld(C), _dp(workspace),
                              _stream_handle(stream)), "spmm_bcsr_run")


def wcsr_run(plan: Plan, B, C, workspace=None, stream=None):
    _run_checks(plan, B, C, workspace)
    _check(_lib.spmm_wcsr_run(plan.handle, _dp(B), _ld(B), _dp(C), _ld(C), _dp(workspace),
                              _stream_handle(stream)), "spmm_wcsr_run")


def wcsr_run_noalloc(plan: Plan, B, C, stream=None):
    """spmm_wcsr_run_noalloc: the WCSR run with the library's static partial-tile
    scratch instead of a workspace (allocates nothing; runs on one GPU must not
    overlap)."""
    _run_checks(plan, B, C, None, check_workspace=False)
    _check(_lib.spmm_wcsr_run_noalloc(plan.handle, _dp(B), _ld(B), _dp(C), _ld(C),
                                      _stream_handle(stream)), "spmm_wcsr_run_noalloc")


# --------------------------------------------------------------------------
# convenience: a device-resident sparse matrix with its plan
# --------------------------------------------------------------------------

_TORCH_C = {"fp32": "float32", "bf16": "bfloat16", "fp16": "float16"}


class DeviceSparse:
    """Builds BCSR or WCSR on the host (native builders), copies the arrays to
    the device, makes the plan and a workspace.  ``run(B, C)`` enqueues C = A*B."""

    def __init__(self, fmt: str, m: int, k: int, N: int, row_ptr, col_idx, values, b_row: int,
                 b_col: int, ab_dtype: str, c_dtype: str, device="cuda", split_cols: int = 0,
                 options=None):
        import torch
        self.fmt, self.m, self.k, self.N = fmt, int(m), int(k), int(N)
        self.ab_dtype, self.c_dtype = ab_dtype, c_dtype
        self.b_row, self.b_col = int(b_row), int(b_col)
        self.code_bytes = 1 if ab_dtype == "fp8" else 2
        if fmt == "bcsr":
            ptr, idx, vals = csr_to_bcsr(m, k, row_ptr, col_idx, values, b_row, b_col,
                                         self.code_bytes)
        elif self.code_bytes == 1:
            raise ValueError("WCSR holds 16-bit values only")
        elif fmt == "wcsr":
            ptr, idx, vals = csr_to_wcsr(m, k, row_ptr, col_idx, values, b_row, b_col)
        else:
            raise ValueError(fmt)
        self.h_ptr, self.h_idx, self.h_vals = ptr, idx, vals
        self.d_idx = torch.from_numpy(idx.copy()).to(device) if idx.size else \
            torch.empty(4, dtype=torch.int32, device=device)
        vt = (np.uint8, torch.uint8) if self.code_bytes == 1 else (np.int16, torch.int16)
        self.d_vals = torch.from_numpy(vals.view(vt[0]).copy()).to(device) if vals.size else \
            torch.empty(16, dtype=vt[1], device=device)
        self.device, self.split_cols = device, int(split_cols)
        self.replan(options)

    def replan(self, options=None):
        """(Re)makes the plan, with ``options`` (dict of PlanOptions fields to
        pin, None: automatic), and its workspace."""
        import torch
        if getattr(self, "plan", None) is not None:
            self.plan.destroy()
        if self.fmt == "bcsr":
            self.plan = bcsr_plan(self.m, self.k, self.N, self.b_row, self.b_col, self.h_ptr,
                                  self.d_idx, self.d_vals, self.ab_dtype, self.c_dtype, options)
        else:
            self.plan = wcsr_plan(self.m, self.k, self.N, self.b_row, self.b_col, self.h_ptr,
                                  self.d_idx, self.d_vals, self.ab_dtype, self.c_dtype,
                                  self.split_cols, options)
        nbytes = self.plan.workspace_bytes
        self.workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32,
                                     device=self.device) if nbytes else None
        self._ws_stream = None
        return self

    def tune(self, B, C, stream=None, reps=0, options=None):
        """Replaces the plan by a tuned one (spmm_*_plan_tuned, timed on B and C;
        C is overwritten) and makes its workspace.  Returns the options the
        tuned plan was made with."""
        import torch
        if self.fmt == "bcsr":
            plan, chosen = bcsr_plan_tuned(self.m, self.k, self.N, self.b_row, self.b_col,
                                           self.h_ptr, self.d_idx, self.d_vals, B, C,
                                           self.ab_dtype, self.c_dtype, options, stream, reps)
        else:
            plan, chosen = wcsr_plan_tuned(self.m, self.k, self.N, self.b_row, self.b_col,
                                           self.h_ptr, self.d_idx, self.d_vals, B, C,
                                           self.ab_dtype, self.c_dtype, self.split_cols,
                                           options, stream, reps)
        self.plan.destroy()
        self.plan = plan
        nbytes = self.plan.workspace_bytes
        self.workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32,
                                     device=self.device) if nbytes else None
        self._ws_stream = None
        return chosen

    @property
    def stored_entries(self) -> int:
        return int(self.h_vals.size)

    def new_c(self, device="cuda", padded: bool = False):
        """Uninitialised C (m x N); ``padded`` allocates rows of recommended_ld
        elements and returns the m x N view."""
        import torch
        dt = getattr(torch, _TORCH_C[self.c_dtype])
        if not padded:
            return torch.empty((self.m, self.N), dtype=dt, device=device)
        ld = recommended_ld(self.N, torch.empty(0, dtype=dt).element_size())
        return torch.empty((self.m, ld), dtype=dt, device=device)[:, :self.N]

    def device_b(self, codes: np.ndarray, device="cuda", padded: bool = False):
        """Copies host codes of B (k x N; 16-bit, or 8-bit for FP8) to the device
        (padded rows optionally)."""
        import torch
        vt = (np.uint8, torch.uint8) if self.code_bytes == 1 else (np.int16, torch.int16)
        src = torch.from_numpy(_codes8(codes) if self.code_bytes == 1 else
                               np.ascontiguousarray(codes).view(vt[0]))
        if not padded:
            return src.to(device)
        ld = recommended_ld(self.N, self.code_bytes)
        out = torch.empty((self.k, ld), dtype=vt[1], device=device)[:, :self.N]
        out.copy_(src)
        return out

    def run(self, B, C, stream=None, workspace=None):
        """Enqueues C = A * B on `stream` (the current stream if None).  The
        object owns one workspace; runs that may overlap (on different
        streams) each need their own, passed as `workspace`.  Without one, a
        plan that uses its workspace (split windows) refuses a stream other
        than the one of its first run."""
        if workspace is None:
            workspace = self.workspace
            if workspace is not None:
                h = _stream_handle(stream).value
                if self._ws_stream is None:
                    self._ws_stream = h
                elif h != self._ws_stream:
                    raise ValueError("this plan's own workspace is in use by another stream; "
                                     "pass a workspace of %d bytes for this one"
                                     % self.plan.workspace_bytes)
        (bcsr_run if self.fmt == "bcsr" else wcsr_run)(self.plan, B, C, workspace, stream)
        return C

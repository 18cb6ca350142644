"""Oracle implementation (test infrastructure only; see the package docstring).

Every function here is written from the AsyncSparse paper's definitions; the
sparse-format encoders are plain numpy scatters of the definition, not a copy
of any kernel-side logic.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(_HERE, "spmm_oracle.c")
ORACLE_LIB = os.path.join(_HERE, "liboracle.so")

_DTYPES = {"fp16": 0, "bf16": 1, "fp8": 3}


def build_oracle(force: bool = False) -> str:
    """Compile the C oracle with the host C compiler (no GPU code involved)."""
    if force or not os.path.exists(ORACLE_LIB) or \
            os.path.getmtime(ORACLE_LIB) < os.path.getmtime(ORACLE_SRC):
        tmp = ORACLE_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread",
                               ORACLE_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, ORACLE_LIB)
    return ORACLE_LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_oracle())
        i64, i32p, u16p, f64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_decode16.restype = ctypes.c_double
        lib.oracle_decode16.argtypes = [ctypes.c_uint16, ctypes.c_int]
        lib.oracle_decode16_array.restype = None
        lib.oracle_decode16_array.argtypes = [u16p, i64, ctypes.c_int, f64p]
        lib.oracle_spmm.restype = ctypes.c_int
        lib.oracle_spmm.argtypes = [i64, i64, i64, i64, i32p, i32p, u16p, u16p, ctypes.c_int,
                                    ctypes.c_void_p, i64, f64p, f64p, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def decode16(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every 16-bit code (binary16 or bfloat16)."""
    c = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_decode16_array(_ptr(c), c.size, _DTYPES[dtype], _ptr(out))
    return out


def spmm(m: int, k: int, N: int, rows: np.ndarray, cols: np.ndarray, a_codes: np.ndarray,
         b_codes: np.ndarray, dtype: str, out_rows: Optional[np.ndarray] = None,
         nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 ``(C, Bound)`` for the requested output rows (all rows by default).

    ``rows, cols, a_codes`` are COO triplets of A (any order; duplicates add up);
    ``b_codes`` is B, ``k x N`` row-major.  ``Bound = |A| * |B|`` on the same rows."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    a = np.ascontiguousarray(a_codes, dtype=np.uint16)
    b = np.ascontiguousarray(b_codes, dtype=np.uint16)
    if not (rows.size == cols.size == a.size):
        raise ValueError("triplet arrays differ in length")
    if b.size != int(k) * int(N):
        raise ValueError("B must hold k*N codes")
    if out_rows is None:
        orow = None
        n_out = int(m)
    else:
        orow = np.ascontiguousarray(out_rows, dtype=np.int64)
        n_out = orow.size
    C = np.empty((n_out, int(N)), dtype=np.float64)
    Bd = np.empty((n_out, int(N)), dtype=np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = _load().oracle_spmm(int(m), int(k), int(N), rows.size, _ptr(rows), _ptr(cols), _ptr(a), _ptr(b),
                             _DTYPES[dtype], None if orow is None else _ptr(orow), n_out,
                             _ptr(C), _ptr(Bd), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_spmm failed with code %d" % rc)
    return C, Bd


# unit roundoff of the 16-bit output formats (8 and 11 significant bits)
OUTPUT_ROUNDOFF = {"fp32": 0.0, "bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def within_tolerance(c_test: np.ndarray, c_ref: np.ndarray, bound: np.ndarray, tol: float = 2e-3,
                     out_dtype: str = "fp32"):
    """Acceptance test, elementwise, C_test finite:

        |C_test - C_ref| <= tol * Bound + u_out * |C_ref|

    ``tol * Bound`` (Bound = sum |a||b|) covers fp16/bf16 products accumulated in
    fp32; ``u_out`` is the unit roundoff of a 16-bit C (one final rounding to
    nearest, 2^-8 for bfloat16, 2^-11 for binary16, 0 for an fp32 C).
    Where Bound is 0 (no product contributes) C_test must be exactly 0.
    Returns ``(ok, worst_ratio, worst_index)``; ratio = tol * |diff| / allowed, which is
    |diff| / Bound for an fp32 C (acceptance: ratio <= tol)."""
    c_test = np.asarray(c_test, dtype=np.float64)
    diff = np.abs(c_test - c_ref)
    allowed = tol * bound + OUTPUT_ROUNDOFF[out_dtype] * np.abs(c_ref)
    bad = ~np.isfinite(c_test) | (diff > allowed)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allowed > 0, diff / np.where(allowed > 0, allowed, 1.0) * tol,
                         np.where(diff > 0, np.inf, 0.0))
    ratio = np.where(np.isfinite(c_test), ratio, np.inf)
    if ratio.size == 0:
        return True, 0.0, None
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return (not bool(bad.any())), float(ratio[worst]), tuple(int(x) for x in worst)


def dense_bruteforce(m: int, k: int, N: int, rows, cols, a_vals, b_vals):
    """Dense A from the triplets, then the textbook triple loop (pure Python).
    Tiny inputs only."""
    A = [[0.0] * k for _ in range(m)]
    for i, j, v in zip(rows, cols, a_vals):
        A[int(i)][int(j)] += float(v)
    C = [[0.0] * N for _ in range(m)]
    for i in range(m):
        for n in range(N):
            s = 0.0
            for j in range(k):
                s += A[i][j] * float(b_vals[j][n])
            C[i][n] = s
    return np.array(C, dtype=np.float64).reshape(m, N)


# --------------------------------------------------------------------------
# sparse formats (Section II-C and Fig. 2)
# --------------------------------------------------------------------------

def _coo_rows(m: int, row_ptr: np.ndarray) -> np.ndarray:
    return np.repeat(np.arange(m, dtype=np.int64), np.diff(np.asarray(row_ptr, dtype=np.int64)))


def encode_bcsr(m: int, k: int, row_ptr, col_idx, vals, b_row: int, b_col: int):
    """BCSR: tile A into b_row x b_col blocks; keep every block holding at least
    one (structural) entry, as a dense row-major tile with +0 elsewhere; blocks of
    a block row in increasing block-column order.
    Returns ``(block_row_ptr int32[ceil(m/b_row)+1], block_col_idx int32[nnz_blocks],
    blocks uint16[nnz_blocks*b_row*b_col])``."""
    rows = _coo_rows(m, row_ptr)
    cols = np.asarray(col_idx, dtype=np.int64)
    nbr = -(-m // b_row)
    nbc = max(1, -(-k // b_col))
    key = (rows // b_row) * nbc + cols // b_col
    ukeys = np.unique(key)
    per_row = np.bincount(ukeys // nbc, minlength=nbr) if nbr > 0 else np.zeros(0, np.int64)
    block_row_ptr = np.concatenate([[0], np.cumsum(per_row)]).astype(np.int32)
    block_col_idx = (ukeys % nbc).astype(np.int32)
    bsz = b_row * b_col
    blocks = np.zeros(ukeys.size * bsz, dtype=np.uint16)
    bidx = np.searchsorted(ukeys, key)
    blocks[bidx * bsz + (rows % b_row) * b_col + cols % b_col] = np.asarray(vals, dtype=np.uint16)
    return block_row_ptr, block_col_idx, blocks


def decode_bcsr(m: int, k: int, block_row_ptr, block_col_idx, blocks, b_row: int, b_col: int):
    """Nonzero codes of a BCSR matrix as COO ``(rows, cols, codes)`` sorted by
    (row, col).  Raises if a nonzero sits outside the m x k matrix."""
    brp = np.asarray(block_row_ptr, dtype=np.int64)
    nblk = int(brp[-1]) if brp.size else 0
    bsz = b_row * b_col
    bl = np.asarray(blocks, dtype=np.uint16)[: nblk * bsz].reshape(nblk, b_row, b_col)
    brow = np.repeat(np.arange(brp.size - 1, dtype=np.int64), np.diff(brp))
    b, r, c = np.nonzero(bl)
    rows = brow[b] * b_row + r
    cols = np.asarray(block_col_idx, dtype=np.int64)[b] * b_col + c
    if rows.size and (rows.max() >= m or cols.max() >= k):
        raise ValueError("nonzero outside the matrix")
    order = np.lexsort((cols, rows))
    return rows[order], cols[order], bl[b, r, c][order]


def encode_wcsr(m: int, k: int, row_ptr, col_idx, vals, b_row: int, b_col: int):
    """WCSR: group rows into windows of b_row; a window keeps the sorted union of
    the column indices of its rows, padded with -1 to a multiple of b_col; the
    window's values form a dense b_row x W tile (W = padded union width), stored
    row-major and contiguous per window, window w starting at element
    ``b_row * window_row_ptr[w]``.
    Returns ``(window_row_ptr int32[ceil(m/b_row)+1], window_col_idx int32[P],
    values uint16[b_row*P])``."""
    rows = _coo_rows(m, row_ptr)
    cols = np.asarray(col_idx, dtype=np.int64)
    nw = -(-m // b_row)
    kk = max(1, k)
    w = rows // b_row
    key = w * kk + cols
    ukeys = np.unique(key)
    uw = ukeys // kk
    n_w = np.bincount(uw, minlength=nw) if nw > 0 else np.zeros(0, np.int64)
    W_w = -(-n_w // b_col) * b_col
    wptr = np.concatenate([[0], np.cumsum(W_w)]).astype(np.int64)
    first = np.concatenate([[0], np.cumsum(n_w)])[:-1] if nw > 0 else np.zeros(0, np.int64)
    rank = np.arange(ukeys.size, dtype=np.int64) - first[uw]
    P = int(wptr[-1])
    window_col_idx = np.full(P, -1, dtype=np.int32)
    window_col_idx[wptr[uw] + rank] = (ukeys % kk).astype(np.int32)
    values = np.zeros(b_row * P, dtype=np.uint16)
    ent_rank = rank[np.searchsorted(ukeys, key)]
    values[b_row * wptr[w] + (rows - w * b_row) * W_w[w] + ent_rank] = np.asarray(vals, dtype=np.uint16)
    return wptr.astype(np.int32), window_col_idx, values


def decode_wcsr(m: int, k: int, window_row_ptr, window_col_idx, values, b_row: int):
    """Nonzero codes of a WCSR matrix as COO ``(rows, cols, codes)`` sorted by
    (row, col).  Raises if a nonzero sits under a pad column or outside A."""
    wptr = np.asarray(window_row_ptr, dtype=np.int64)
    idx = np.asarray(window_col_idx, dtype=np.int64)
    vals = np.asarray(values, dtype=np.uint16)
    R, C, V = [], [], []
    for w in range(wptr.size - 1):
        p0, p1 = int(wptr[w]), int(wptr[w + 1])
        W = p1 - p0
        if W == 0:
            continue
        tile = vals[b_row * p0: b_row * p1].reshape(b_row, W)
        r, p = np.nonzero(tile)
        if r.size == 0:
            continue
        c = idx[p0 + p]
        if np.any(c < 0):
            raise ValueError("nonzero under a pad column")
        R.append(w * b_row + r)
        C.append(c)
        V.append(tile[r, p])
    if not R:
        z = np.zeros(0, np.int64)
        return z, z, np.zeros(0, np.uint16)
    rows, cols, codes = np.concatenate(R), np.concatenate(C), np.concatenate(V)
    if rows.max() >= m or cols.max() >= k:
        raise ValueError("nonzero outside the matrix")
    order = np.lexsort((cols, rows))
    return rows[order], cols[order], codes[order]


def wcsr_tasks(window_row_ptr, T: int):
    """Window splitting (Section III-C): a window of W <= T packed columns is one
    task that writes C directly (slot -1); a longer window becomes ceil(W / T)
    tasks of T columns (the last one shorter), each writing its own partial slot,
    and one merge record ``(window, first_slot, n_slots)``.  Empty windows are one
    empty task (their rows of C become zero).
    Returns ``(tasks int32[n,4] = (window, col_begin, col_end, slot),
    merges int32[s,3])``."""
    wptr = np.asarray(window_row_ptr, dtype=np.int64)
    tasks, merges = [], []
    slot = 0
    for w in range(wptr.size - 1):
        p0, p1 = int(wptr[w]), int(wptr[w + 1])
        if p1 - p0 <= T:
            tasks.append((w, p0, p1, -1))
            continue
        n = -(-(p1 - p0) // T)
        merges.append((w, slot, n))
        for t in range(n):
            tasks.append((w, p0 + t * T, min(p1, p0 + (t + 1) * T), slot + t))
        slot += n
    return (np.array(tasks, dtype=np.int32).reshape(-1, 4),
            np.array(merges, dtype=np.int32).reshape(-1, 3))


def padded_width(N: int, BN: int) -> int:
    """Columns actually computed when N is padded up to a multiple of the tile
    width BN (Section IV-C)."""
    return int(math.ceil(N / BN) * BN)


def fill_ratio(nnz: int, nnz_blocks: int, b_row: int, b_col: int) -> float:
    """Fraction of stored block entries that are real nonzeros (Section II-C)."""
    return nnz / float(nnz_blocks * b_row * b_col) if nnz_blocks else 0.0

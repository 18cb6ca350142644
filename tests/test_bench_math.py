"""The benchmark's roofline arithmetic (flops and algorithmic bytes of one SpMM,
as the measurement defines them: stored A values, format metadata, each
referenced B row once, C once), on hand-worked tiny formats.  CPU only."""

import types

import numpy as np

import bench


def _problem(fmt, m, k, N, nnz, b_row, b_col, c_dtype="fp32", ab_dtype="fp16"):
    return types.SimpleNamespace(fmt=fmt, m=m, k=k, N=N, nnz=nnz, b_row=b_row, b_col=b_col,
                                 c_dtype=c_dtype, ab_dtype=ab_dtype)


def test_wcsr_bytes_and_flops_by_hand():
    # two windows of 16 rows (m = 32, k = 40), b_col = 8:
    # window 0 uses columns {1, 3, 4} -> padded to 8 (5 pads), window 1 uses
    # {3, 20, 21, 22, 23, 24, 25, 26, 27} -> padded to 16 (7 pads)
    idx = np.array([1, 3, 4] + [-1] * 5 + [3, 20, 21, 22, 23, 24, 25, 26, 27] + [-1] * 7, np.int32)
    ptr = np.array([0, 8, 24], np.int32)
    P = 24
    A = types.SimpleNamespace(stored_entries=16 * P, h_ptr=ptr, h_idx=idx)
    p = _problem("wcsr", 32, 40, 64, nnz=50, b_row=16, b_col=8)
    got = bench.algorithmic(p, A)
    # A values 2*16*24 = 768, indices 4*24 = 96, row pointer 4*3 = 12,
    # distinct B rows {1,3,4,20..27} = 11 -> 2*64*11 = 1408, C 4*32*64 = 8192
    assert got["bytes_alg"] == 768 + 96 + 12 + 1408 + 8192
    assert got["b_rows_referenced"] == 11
    assert got["flops_true"] == 2 * 50 * 64
    assert got["flops_stored"] == 2 * 16 * 24 * 64


def test_bcsr_bytes_with_a_ragged_last_block_column():
    # k = 20 with 8-wide block columns: block column 2 covers rows 16..19 only.
    # Block row 0 holds block columns {0, 2}, block row 1 holds {2}; bf16 C.
    ptr = np.array([0, 2, 3], np.int32)
    idx = np.array([0, 2, 2], np.int32)
    A = types.SimpleNamespace(stored_entries=3 * 16 * 8, h_ptr=ptr, h_idx=idx)
    p = _problem("bcsr", 32, 20, 16, nnz=100, b_row=16, b_col=8, c_dtype="bf16", ab_dtype="bf16")
    got = bench.algorithmic(p, A)
    # A 2*384 = 768, block indices 4*3 = 12, row pointer 4*3 = 12,
    # B rows 0..7 and 16..19 = 12 -> 2*16*12 = 384, C 2*32*16 = 1024
    assert got["b_rows_referenced"] == 12
    assert got["bytes_alg"] == 768 + 12 + 12 + 384 + 1024
    assert got["flops_stored"] == 2 * 384 * 16


def test_roofline_time_takes_the_larger_bound():
    p = _problem("bcsr", 1, 1, 1, nnz=1, b_row=16, b_col=16)
    # 2.5e15 flop/s and 8e12 B/s: 5e12 flop -> 2 ms; 8e9 bytes -> 1 ms
    alg = {"flops_stored": 5e12, "bytes_alg": 8e9}
    assert abs(bench.roofline_time(p, alg) - 2e-3) < 1e-12
    alg = {"flops_stored": 5e11, "bytes_alg": 8e9}
    assert abs(bench.roofline_time(p, alg) - 1e-3) < 1e-12


def test_traffic_key_ignores_comments_but_not_code():
    # the key of a traffic record follows the code: comments, blank lines and
    # indentation do not count, literals that look like comments do
    src = 'int f(int x) {\n    return x + 1; // one\n}\n'
    assert bench.code_only(src) == bench.code_only('/* doc */\nint f(int x) {\n\n  return x + 1;\n}')
    assert bench.code_only(src) != bench.code_only(src.replace("x + 1", "x + 2"))
    lit = 'const char *s = "a // b /* c */"; char q = \'/\';'
    assert bench.code_only(lit) == lit
    assert bench.code_only('a /* x */ b') == 'a   b'
    assert len(bench.kernel_source_sha256()) == 64

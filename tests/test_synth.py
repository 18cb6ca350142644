"""The seeded generators: determinism and the recipe's structural promises."""

import hashlib

import numpy as np
import pytest

import synth


def _digest(p):
    h = hashlib.sha256()
    for a in (p.row_ptr, p.col_idx, p.vals, p.B):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def _check_csr(p):
    assert p.row_ptr.dtype == np.int32 and p.col_idx.dtype == np.int32
    assert p.row_ptr[0] == 0 and p.row_ptr[-1] == p.nnz and np.all(np.diff(p.row_ptr) >= 0)
    rows = p.coo_rows()
    same_row = rows[1:] == rows[:-1]
    assert np.all(np.diff(p.col_idx)[same_row] > 0)      # sorted, unique
    assert p.col_idx.min(initial=0) >= 0 and p.col_idx.max(initial=-1) < p.k
    assert np.all((p.vals & 0x7FFF) != 0)                  # structure == nonzero values
    assert p.B.shape == (p.k, p.N) and p.B.dtype == np.uint16


def test_same_seed_same_arrays_other_seed_differs():
    a, b, c = synth.config1(0), synth.config1(0), synth.config1(1)
    assert _digest(a) == _digest(b) != _digest(c)
    r1 = synth.random_problem(40, 50, 8, 0.1, seed=3)
    r2 = synth.random_problem(40, 50, 8, 0.1, seed=3)
    assert _digest(r1) == _digest(r2)


def test_config1_recipe():
    p = synth.config1()
    _check_csr(p)
    assert (p.m, p.k, p.N, p.b_row, p.b_col) == (256, 256, 64, 16, 16)
    blocks = {(int(r) // 16, int(c) // 16) for r, c in zip(p.coo_rows(), p.col_idx)}
    assert len(blocks) == 26 and p.nnz == 26 * 256


def test_config4_recipe_small_n():
    for which, keep in (("gate", 6), ("down", 30)):
        p = synth.config4(which, N=64)
        _check_csr(p)
        rows = p.coo_rows()
        per = {}
        for r, c in zip(rows[::64], p.col_idx[::64]):
            per.setdefault(int(r) // 64, set()).add(int(c) // 64)
        assert all(len(v) == keep for v in per.values()) and len(per) == p.m // 64


def test_config3_specs_ranges():
    specs = synth.config3_specs()
    assert len(specs) == 32
    for j, (m, mu, banded) in enumerate(specs):
        assert 8192 <= m <= 524288 and 4 <= mu <= 256 and banded == (j % 2 == 0)


@pytest.mark.parametrize("j", [0, 3])
def test_config3_small_members(j):
    p = synth.config3_matrix(j, 32)
    _check_csr(p)
    mean = p.nnz / p.m
    assert abs(mean - p.meta["target_mean"]) / p.meta["target_mean"] < 0.05
    if p.meta["banded"]:
        bw = int(np.floor(0.01 * p.m))
        assert np.all(np.abs(p.col_idx - p.coo_rows()) <= bw)


def test_random_and_block_problems_are_valid():
    for s in range(4):
        _check_csr(synth.random_problem(33, 47, 16, 0.2, seed=s, empty_row_frac=0.3))
        _check_csr(synth.block_problem(70, 90, 16, 16, 16, 0.3, seed=s, entry_density=0.5))


def test_bf16_conversion_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    assert synth.bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020]

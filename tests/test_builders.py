"""Host-side format builders and the split rule of the native library, byte for
byte against the oracle's encoders (integer work: bit-exact).  CPU only."""

import numpy as np
import pytest

import oracle
import synth
import window_spmm_amd as ws
from conftest import load_fig2


def _same(a, b):
    return all(np.array_equal(np.asarray(x), np.asarray(y)) and np.asarray(x).dtype == np.asarray(y).dtype
               for x, y in zip(a, b))


def _both(p, br, bc):
    nb = ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc)
    ob = oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc)
    nw = ws.csr_to_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc)
    ow = oracle.encode_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc)
    return nb, ob, nw, ow


def test_fig2_through_the_abi():
    spec = load_fig2()
    e = sorted(spec["e"])
    m, k = spec["m"], spec["k"]
    rows = np.array([x[0] for x in e])
    ptr = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=m))]).astype(np.int32)
    cols = np.array([x[1] for x in e], np.int32)
    vals = synth.fp16_bits(np.array([x[2] for x in e], np.float64))
    brp, bci, _ = ws.csr_to_bcsr(m, k, ptr, cols, vals, spec["b_row"], spec["b_col"])
    wrp, wci, _ = ws.csr_to_wcsr(m, k, ptr, cols, vals, spec["b_row"], spec["b_col"])
    assert brp.tolist() == spec["block_row_ptr"] and bci.tolist() == spec["block_col_idx"]
    assert wrp.tolist() == spec["window_row_ptr"] and wci.tolist() == spec["window_col_idx"]


@pytest.mark.parametrize("seed", range(8))
def test_builders_match_oracle_fuzz(seed):
    g = np.random.default_rng(seed)
    m, k = int(g.integers(0, 300)), int(g.integers(1, 400))
    br = int(g.choice([1, 2, 8, 16, 32, 64]))
    bc = int(g.choice([1, 4, 8, 16, 64]))
    p = synth.random_problem(m, k, 8, float(g.uniform(0.001, 0.2)), seed=seed,
                             empty_row_frac=float(g.uniform(0, 0.5)))
    nb, ob, nw, ow = _both(p, br, bc)
    assert _same(nb, ob) and _same(nw, ow)


def test_builders_match_oracle_block_patterns():
    for s, (br, bc) in enumerate([(16, 16), (64, 64), (32, 16), (64, 32)]):
        p = synth.block_problem(300, 260, 8, br, bc, 0.2, seed=s, entry_density=0.6)
        nb, ob, nw, ow = _both(p, br, bc)
        assert _same(nb, ob) and _same(nw, ow)


def test_bcsr8_builder_matches_oracle():
    """The 8-bit builder (FP8 E4M3 codes) lays out blocks exactly as the 16-bit
    one: the oracle's encoding with every code narrowed to a byte."""
    for s, (br, bc) in enumerate([(64, 64), (16, 16), (32, 8)]):
        p = synth.block_problem(300, 260, 8, br, bc, 0.2, seed=s, ab_dtype="fp8",
                                entry_density=0.6)
        assert int(p.vals.max()) <= 255
        ptr, idx, blk = ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc,
                                       code_bytes=1)
        optr, oidx, oblk = oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc)
        assert blk.dtype == np.uint8
        assert np.array_equal(ptr, optr) and np.array_equal(idx, oidx)
        assert np.array_equal(blk, oblk.astype(np.uint8))
    with pytest.raises(ValueError):
        ws.csr_to_bcsr(2, 2, [0, 1, 1], [0], np.array([300], np.uint16), 16, 16, code_bytes=1)


def test_one_by_one_is_csr():
    p = synth.random_problem(64, 90, 8, 0.1, seed=4)
    brp, bci, blk = ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 1, 1)
    assert np.array_equal(brp, p.row_ptr) and np.array_equal(bci, p.col_idx) and np.array_equal(blk, p.vals)
    wrp, wci, wv = ws.csr_to_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 1, 1)
    assert np.array_equal(wrp, p.row_ptr) and np.array_equal(wci, p.col_idx) and np.array_equal(wv, p.vals)


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg4_gate", "cfg4_down"])
def test_builders_match_oracle_on_configs(name, cfg2):
    p = {"cfg1": lambda: synth.config1(),
         "cfg2": lambda: cfg2,
         "cfg4_gate": lambda: synth.config4("gate", N=8, with_b=False),
         "cfg4_down": lambda: synth.config4("down", N=8, with_b=False)}[name]()
    if p.fmt == "bcsr":
        ob = oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col)
        nb = ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col)
        assert _same(nb, ob)
    nw = ws.csr_to_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 16, 8)
    ow = oracle.encode_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 16, 8)
    assert _same(nw, ow)


@pytest.mark.slow
def test_builders_match_oracle_config5():
    p = synth.config5(with_b=False)
    nb = ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 64, 64)
    ob = oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 64, 64)
    assert _same(nb, ob)
    assert nb[0][-1] == p.meta["kept_blocks"]


def test_decode_of_native_encode_is_identity():
    p = synth.random_problem(333, 257, 8, 0.03, seed=9, empty_row_frac=0.2)
    rows = p.coo_rows()
    brp, bci, blk = ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 32, 16)
    r, c, v = oracle.decode_bcsr(p.m, p.k, brp, bci, blk, 32, 16)
    assert np.array_equal(r, rows) and np.array_equal(c, p.col_idx) and np.array_equal(v, p.vals)
    wrp, wci, wv = ws.csr_to_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 16, 8)
    r, c, v = oracle.decode_wcsr(p.m, p.k, wrp, wci, wv, 16)
    assert np.array_equal(r, rows) and np.array_equal(c, p.col_idx) and np.array_equal(v, p.vals)


@pytest.mark.parametrize("T", [32, 64, 256, 4096])
def test_split_matches_oracle(T, cfg2):
    p = cfg2
    wrp, _, _ = ws.csr_to_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 16, 8)
    nt, nm = ws.wcsr_split(wrp, T)
    ot, om = oracle.wcsr_tasks(wrp, T)
    assert np.array_equal(nt, ot) and np.array_equal(nm, om)


def test_split_hand_example():
    t, m = ws.wcsr_split(np.array([0, 8, 8, 40, 48], np.int32), 32)
    assert t.tolist() == [[0, 0, 8, -1], [1, 8, 8, -1], [2, 8, 40, -1], [3, 40, 48, -1]]
    assert m.shape == (0, 3)
    t, m = ws.wcsr_split(np.array([0, 8, 8, 72, 80], np.int32), 32)
    assert t.tolist() == [[0, 0, 8, -1], [1, 8, 8, -1], [2, 8, 40, 0], [2, 40, 72, 1], [3, 72, 80, -1]]
    assert m.tolist() == [[2, 0, 2]]


# ---- error paths (forced from the host) ----

def _err(fn):
    with pytest.raises(ws.SpmmError) as e:
        fn()
    return e.value.code


def test_builder_rejects_bad_csr():
    ptr = np.array([0, 2, 3], np.int32)
    assert _err(lambda: ws.csr_to_bcsr(2, 5, ptr, np.array([3, 1, 0], np.int32),
                                       np.ones(3, np.uint16), 2, 2)) == ws.ERR_BAD_FORMAT
    assert _err(lambda: ws.csr_to_wcsr(2, 5, ptr, np.array([1, 1, 0], np.int32),
                                       np.ones(3, np.uint16), 2, 2)) == ws.ERR_BAD_FORMAT
    assert _err(lambda: ws.csr_to_wcsr(2, 5, ptr, np.array([1, 2, 5], np.int32),
                                       np.ones(3, np.uint16), 2, 2)) == ws.ERR_BAD_FORMAT
    assert _err(lambda: ws.csr_to_bcsr(2, 5, np.array([0, 2, 1], np.int32), np.array([1, 2], np.int32),
                                       np.ones(2, np.uint16), 2, 2)) == ws.ERR_BAD_FORMAT
    assert _err(lambda: ws.csr_to_bcsr(2, 5, ptr, np.array([1, 2, 0], np.int32),
                                       np.ones(3, np.uint16), 0, 2)) == ws.ERR_INVALID_ARGUMENT


def test_split_rejects_bad_t():
    assert _err(lambda: ws.wcsr_split(np.array([0, 8], np.int32), 48)) == ws.ERR_INVALID_ARGUMENT
    assert _err(lambda: ws.wcsr_split(np.array([0, 8, 0], np.int32), 32)) == ws.ERR_BAD_FORMAT


# --------------------------------------------------------------------------
# reverse Cuthill-McKee and the symmetric permutation (Section IV-A)
# --------------------------------------------------------------------------

def _random_square(n, density, seed, components=1):
    """Unsymmetric random pattern; with components > 1, block diagonal (no
    edges between the parts) plus a few isolated vertices."""
    rng = np.random.default_rng(seed)
    dense = np.zeros((n, n), bool)
    cuts = np.linspace(0, n - 3 if n > 6 else n, components + 1).astype(int)
    for a, b in zip(cuts[:-1], cuts[1:]):
        dense[a:b, a:b] = rng.random((b - a, b - a)) < density
    rows, cols = np.nonzero(dense)
    row_ptr = np.searchsorted(rows, np.arange(n + 1)).astype(np.int32)
    vals = rng.integers(1, 0x7BFF, size=rows.size).astype(np.uint16)
    return row_ptr, cols.astype(np.int32), vals


@pytest.mark.parametrize("n,density,seed,parts", [(1, 0.5, 0, 1), (9, 0.3, 1, 1), (200, 0.02, 2, 1),
                                                  (500, 0.01, 3, 4), (1500, 0.004, 4, 2),
                                                  (800, 0.0005, 5, 1)])
def test_rcm_matches_oracle(n, density, seed, parts):
    rp, ci, v = _random_square(n, density, seed, parts)
    perm = ws.rcm_order(n, rp, ci)
    assert np.array_equal(perm, oracle.rcm_order(n, rp, ci))
    got = ws.csr_permute(n, rp, ci, v, perm)
    want = oracle.permute_symmetric(n, rp, ci, v, perm)
    assert _same(got, want)


def test_rcm_hand_example_through_the_abi():
    # path 1-2-3-4-5-6 with 0 hanging off 3 (worked by hand in the oracle pins)
    rp = np.array([0, 1, 2, 3, 4, 5, 6, 6], np.int32)
    ci = np.array([3, 2, 3, 4, 5, 6], np.int32)
    assert ws.rcm_order(7, rp, ci).tolist() == [1, 2, 0, 3, 4, 5, 6]


def test_rcm_recovers_a_shuffled_band_and_raises_wcsr_fill():
    # banded pattern (half-width 1% of n, like the banded half of the SuiteSparse
    # stand-ins), relabelled at random: RCM brings the union width per window
    # back down (the effect the paper reorders for)
    n, half = 4096, 40
    rng = np.random.default_rng(11)
    i = np.repeat(np.arange(n), 2 * half + 1)
    j = i + np.tile(np.arange(-half, half + 1), n)
    keep = (j >= 0) & (j < n) & (rng.random(i.size) < 0.25)
    i, j = i[keep], j[keep]
    orp = np.searchsorted(i, np.arange(n + 1)).astype(np.int32)
    original = ws.csr_to_wcsr(n, n, orp, j.astype(np.int32), np.ones(j.size, np.uint16), 16, 8)[0][-1]
    lab = rng.permutation(n)
    dense_rows, dense_cols = lab[i], lab[j]
    order = np.lexsort((dense_cols, dense_rows))
    r, c = dense_rows[order], dense_cols[order]
    rp = np.searchsorted(r, np.arange(n + 1)).astype(np.int32)
    ci = c.astype(np.int32)
    v = np.ones(ci.size, np.uint16) * 0x3C00
    before = ws.csr_to_wcsr(n, n, rp, ci, v, 16, 8)[0][-1]
    perm = ws.rcm_order(n, rp, ci)
    prp, pci, pv = ws.csr_permute(n, rp, ci, v, perm)
    after = ws.csr_to_wcsr(n, n, prp, pci, pv, 16, 8)[0][-1]
    # shuffled, a window's union is nearly all of its rows' entries; after RCM it
    # is about the original band's union again
    assert after * 3 < before
    assert after <= 1.25 * original
    assert oracle.bandwidth(n, prp, pci) <= 4 * half


def test_rcm_and_permute_reject_bad_input():
    rp = np.array([0, 2, 1], np.int32)
    with pytest.raises(ws.SpmmError, match="BAD_FORMAT"):
        ws.rcm_order(2, rp, np.array([0, 1], np.int32))
    rp = np.array([0, 1, 2], np.int32)
    ci = np.array([1, 0], np.int32)
    v = np.ones(2, np.uint16)
    with pytest.raises(ws.SpmmError, match="INVALID_ARGUMENT"):
        ws.csr_permute(2, rp, ci, v, np.array([0, 0], np.int32))
    with pytest.raises(ws.SpmmError, match="INVALID_ARGUMENT"):
        ws.csr_permute(2, rp, ci, v, np.array([0, 2], np.int32))
    assert ws.rcm_order(0, np.zeros(1, np.int32), np.zeros(0, np.int32)).size == 0

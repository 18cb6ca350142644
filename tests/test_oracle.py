"""Pins for the CPU oracle: each test ties an oracle function to something other
than itself (a library routine, the paper's printed worked example, a closed
form, an invariant or a brute force).  No GPU needed."""

import numpy as np
import pytest

import oracle
import synth
from conftest import load_fig2


def _dense_from_coo(m, k, rows, cols, vals):
    A = np.zeros((m, k), dtype=np.float64)
    np.add.at(A, (np.asarray(rows, np.int64), np.asarray(cols, np.int64)), vals)
    return A


def _run(p: synth.Problem, **kw):
    return oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, p.ab_dtype, **kw)


# --------------------------------------------------------------------------
# 16-bit decoder vs library conversions, all 65536 codes
# --------------------------------------------------------------------------

def test_decode_fp16_matches_numpy_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode16(codes, "fp16")
    lib = codes.view(np.float16).astype(np.float64)
    same = (ours == lib) | (np.isnan(ours) & np.isnan(lib))
    assert same.all()
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_decode_bf16_matches_fp32_upper_half_all_codes():
    codes = np.arange(65536, dtype=np.uint32)
    ours = oracle.decode16(codes.astype(np.uint16), "bf16")
    with np.errstate(invalid="ignore"):
        lib = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    same = (ours == lib) | (np.isnan(ours) & np.isnan(lib))
    assert same.all()


def test_decode_known_values():
    assert oracle.decode16(np.array([0x3C00], np.uint16), "fp16")[0] == 1.0
    assert oracle.decode16(np.array([0x0001], np.uint16), "fp16")[0] == 2.0 ** -24
    assert oracle.decode16(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert oracle.decode16(np.array([0xC000], np.uint16), "bf16")[0] == -2.0
    assert oracle.decode16(np.array([0x0001], np.uint16), "bf16")[0] == 2.0 ** -133


# --------------------------------------------------------------------------
# the product itself
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_spmm_matches_dense_triple_loop(seed, dtype):
    rng = np.random.default_rng(seed)
    m, k, N = int(rng.integers(1, 10)), int(rng.integers(1, 12)), int(rng.integers(1, 7))
    p = synth.random_problem(m, k, N, 0.4, seed=seed, ab_dtype=dtype)
    C, Bd = _run(p, nthreads=2)
    a = oracle.decode16(p.vals, dtype)
    b = oracle.decode16(p.B, dtype).reshape(k, N)
    ref = oracle.dense_bruteforce(m, k, N, p.coo_rows(), p.col_idx, a, b)
    assert np.allclose(C, ref, rtol=1e-12, atol=1e-300)
    absref = oracle.dense_bruteforce(m, k, N, p.coo_rows(), p.col_idx, np.abs(a), np.abs(b))
    assert np.allclose(Bd, absref, rtol=1e-12, atol=1e-300)


def test_spmm_integer_data_is_exact():
    p = synth.random_problem(7, 9, 5, 0.5, seed=3, kind="int")
    C, _ = _run(p)
    a = oracle.decode16(p.vals, "fp16")
    b = oracle.decode16(p.B, "fp16").reshape(9, 5)
    ref = oracle.dense_bruteforce(7, 9, 5, p.coo_rows(), p.col_idx, a, b)
    assert np.array_equal(C, ref)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_spmm_matches_numpy_matmul_medium(dtype):
    p = synth.random_problem(96, 130, 40, 0.07, seed=11, ab_dtype=dtype, empty_row_frac=0.1)
    C, Bd = _run(p)
    A = _dense_from_coo(p.m, p.k, p.coo_rows(), p.col_idx, oracle.decode16(p.vals, dtype))
    B = oracle.decode16(p.B, dtype).reshape(p.k, p.N)
    assert np.all(np.abs(C - A @ B) <= 1e-12 * Bd)
    assert np.allclose(Bd, np.abs(A) @ np.abs(B), rtol=1e-13, atol=0)


def test_identity_gives_b_exactly():
    n, N = 40, 24
    one = synth.fp16_bits(np.ones(n))
    rows = np.arange(n, dtype=np.int32)
    B = synth.make_dense_b(np.random.default_rng(0), n, N, "fp16")
    C, Bd = oracle.spmm(n, n, N, rows, rows, one, B, "fp16")
    assert np.array_equal(C, oracle.decode16(B, "fp16").reshape(n, N))
    assert np.array_equal(Bd, np.abs(C))


def test_zero_matrix_gives_zero():
    B = synth.make_dense_b(np.random.default_rng(1), 10, 8, "bf16")
    z = np.zeros(0, np.int32)
    C, Bd = oracle.spmm(6, 10, 8, z, z, np.zeros(0, np.uint16), B, "bf16")
    assert not C.any() and not Bd.any()


def test_single_entry_scales_one_row():
    B = synth.make_dense_b(np.random.default_rng(2), 5, 16, "fp16")
    a = synth.fp16_bits(np.array([-1.5]))
    C, _ = oracle.spmm(4, 5, 16, np.array([2], np.int32), np.array([3], np.int32), a, B, "fp16")
    b = oracle.decode16(B, "fp16").reshape(5, 16)
    assert np.array_equal(C[2], -1.5 * b[3])
    assert not C[[0, 1, 3]].any()


def test_linear_in_b_exact_on_integers():
    p = synth.random_problem(20, 30, 12, 0.2, seed=4, kind="int")
    g = np.random.default_rng(5)
    b1 = g.integers(-20, 21, size=(30, 12)).astype(np.float64)
    b2 = g.integers(-20, 21, size=(30, 12)).astype(np.float64)
    rows = p.coo_rows()
    c1, _ = oracle.spmm(20, 30, 12, rows, p.col_idx, p.vals, synth.fp16_bits(b1), "fp16")
    c2, _ = oracle.spmm(20, 30, 12, rows, p.col_idx, p.vals, synth.fp16_bits(b2), "fp16")
    c12, _ = oracle.spmm(20, 30, 12, rows, p.col_idx, p.vals, synth.fp16_bits(b1 + b2), "fp16")
    assert np.array_equal(c12, c1 + c2)


def test_duplicate_triplets_add_up():
    B = synth.fp16_bits(np.arange(6, dtype=np.float64).reshape(3, 2))
    a = synth.fp16_bits(np.array([1.0, 2.0]))
    rows = np.array([1, 1], np.int32)
    cols = np.array([2, 2], np.int32)
    C, _ = oracle.spmm(2, 3, 2, rows, cols, a, B, "fp16")
    assert np.array_equal(C[1], np.array([12.0, 15.0]))


def test_row_subset_and_thread_count_do_not_change_values():
    p = synth.random_problem(300, 200, 16, 0.05, seed=8)
    full1, b1 = _run(p, nthreads=1)
    full8, b8 = _run(p, nthreads=8)
    assert np.array_equal(full1, full8) and np.array_equal(b1, b8)
    pick = np.array([299, 0, 17, 17, 150], dtype=np.int64)
    sub, subb = _run(p, out_rows=pick, nthreads=3)
    assert np.array_equal(sub, full1[pick]) and np.array_equal(subb, b1[pick])


def test_rejects_out_of_range_index():
    B = np.zeros((3, 2), np.uint16)
    with pytest.raises(ValueError):
        oracle.spmm(2, 3, 2, np.array([0], np.int32), np.array([3], np.int32),
                    np.array([0x3C00], np.uint16), B, "fp16")


@pytest.mark.parametrize("mistake", ["drop_last", "flip_sign", "swap_b_rows", "transpose_b"])
def test_brute_force_pin_catches_planted_mistakes(mistake):
    """Plant a plausible oracle mistake on the CPU (by feeding the oracle the
    corrupted operand it would effectively use) and check the pin fails."""
    p = synth.random_problem(8, 8, 8, 0.5, seed=21, kind="int")
    a = oracle.decode16(p.vals, "fp16")
    b = oracle.decode16(p.B, "fp16").reshape(8, 8)
    ref = oracle.dense_bruteforce(8, 8, 8, p.coo_rows(), p.col_idx, a, b)
    rows, cols, vals, B = p.coo_rows(), p.col_idx.copy(), p.vals.copy(), p.B.copy()
    if mistake == "drop_last":
        rows, cols, vals = rows[:-1], cols[:-1], vals[:-1]
    elif mistake == "flip_sign":
        vals[0] ^= 0x8000
    elif mistake == "swap_b_rows":
        B = B[[1, 0] + list(range(2, 8))]
    elif mistake == "transpose_b":
        B = np.ascontiguousarray(B.T)
    C, _ = oracle.spmm(8, 8, 8, rows, cols, vals, B, "fp16")
    assert not np.array_equal(C, ref)


# --------------------------------------------------------------------------
# acceptance test
# --------------------------------------------------------------------------

def test_tolerance_accepts_and_rejects():
    ref = np.array([[1.0, -2.0, 0.0]])
    bound = np.array([[10.0, 10.0, 0.0]])
    ok, worst, _ = oracle.within_tolerance(ref + [[0.019, -0.019, 0.0]], ref, bound)
    assert ok and worst < 2e-3
    ok, _, at = oracle.within_tolerance(ref + [[0.021, 0.0, 0.0]], ref, bound)
    assert not ok and at == (0, 0)
    ok, _, at = oracle.within_tolerance(ref + [[0.0, 0.0, 1e-30]], ref, bound)
    assert not ok and at == (0, 2)          # Bound 0 demands an exact zero
    ok, _, _ = oracle.within_tolerance(np.array([[np.nan, -2.0, 0.0]]), ref, bound)
    assert not ok


def test_tolerance_allows_one_rounding_of_a_16bit_output():
    # 16.6877 lies between the bfloat16 neighbours 16.625 and 16.75 (spacing 2^-3);
    # nearest-even gives 16.75, 0.0623 away, more than 2e-3 * Bound when |C| ~ Bound
    ref = np.array([16.687693680636585])
    bound = np.array([23.422590876929462])
    got = oracle.decode16(synth.bf16_bits(ref), "bf16")
    assert got[0] == 16.75
    assert not oracle.within_tolerance(got, ref, bound)[0]
    assert oracle.within_tolerance(got, ref, bound, out_dtype="bf16")[0]
    # the allowance is one rounding, not two
    assert not oracle.within_tolerance(np.array([16.875]), ref, bound, out_dtype="bf16")[0]
    got16 = oracle.decode16(synth.fp16_bits(ref), "fp16")
    assert oracle.within_tolerance(got16, ref, bound * 1e-3, out_dtype="fp16")[0]


# --------------------------------------------------------------------------
# formats: Fig. 2, special cases, round trips, a loop re-implementation
# --------------------------------------------------------------------------

def _fig2_csr(spec):
    e = sorted(spec["e"])
    m = spec["m"]
    rows = np.array([x[0] for x in e])
    cols = np.array([x[1] for x in e], np.int32)
    vals = synth.fp16_bits(np.array([x[2] for x in e], np.float64))
    ptr = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=m))]).astype(np.int32)
    return ptr, cols, vals


def test_fig2_printed_arrays(fig2):
    ptr, cols, vals = _fig2_csr(fig2)
    m, k, br, bc = fig2["m"], fig2["k"], fig2["b_row"], fig2["b_col"]
    brp, bci, blocks = oracle.encode_bcsr(m, k, ptr, cols, vals, br, bc)
    assert brp.tolist() == fig2["block_row_ptr"]
    assert bci.tolist() == fig2["block_col_idx"]
    wrp, wci, wv = oracle.encode_wcsr(m, k, ptr, cols, vals, br, bc)
    assert wrp.tolist() == fig2["window_row_ptr"]
    assert wci.tolist() == fig2["window_col_idx"]
    # storage sizes from the definitions: 5 blocks of 4x4, 12 packed columns x 4 rows
    assert blocks.size == 5 * 16 and wv.size == 4 * 12
    assert oracle.fill_ratio(15, 5, 4, 4) == 15 / 80


def test_one_by_one_blocks_and_windows_are_csr():
    p = synth.random_problem(50, 70, 8, 0.1, seed=5, empty_row_frac=0.2)
    brp, bci, blocks = oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 1, 1)
    assert np.array_equal(brp, p.row_ptr) and np.array_equal(bci, p.col_idx)
    assert np.array_equal(blocks, p.vals)
    wrp, wci, wv = oracle.encode_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 1, 1)
    assert np.array_equal(wrp, p.row_ptr) and np.array_equal(wci, p.col_idx)
    assert np.array_equal(wv, p.vals)


def _loop_bcsr(m, k, ptr, cols, vals, br, bc):
    nbr = -(-m // br)
    blocks = {}
    for i in range(m):
        for t in range(ptr[i], ptr[i + 1]):
            j = int(cols[t])
            blk = blocks.setdefault((i // br, j // bc), [0] * (br * bc))
            blk[(i % br) * bc + j % bc] = int(vals[t])
    rp, ci, data = [0], [], []
    for I in range(nbr):
        for J in sorted(J for (II, J) in blocks if II == I):
            ci.append(J)
            data.extend(blocks[(I, J)])
        rp.append(len(ci))
    return rp, ci, data


def _loop_wcsr(m, k, ptr, cols, vals, br, bc):
    nw = -(-m // br)
    rp, ci, data = [0], [], []
    for w in range(nw):
        rows = range(w * br, min(m, (w + 1) * br))
        union = sorted({int(cols[t]) for i in rows for t in range(ptr[i], ptr[i + 1])})
        W = -(-len(union) // bc) * bc
        tile = [[0] * W for _ in range(br)]
        for i in rows:
            for t in range(ptr[i], ptr[i + 1]):
                tile[i - w * br][union.index(int(cols[t]))] = int(vals[t])
        ci.extend(union + [-1] * (W - len(union)))
        for r in range(br):
            data.extend(tile[r])
        rp.append(rp[-1] + W)
    return rp, ci, data


@pytest.mark.parametrize("seed,m,k,br,bc", [(0, 37, 29, 4, 4), (1, 64, 64, 16, 8), (2, 50, 131, 16, 16),
                                            (3, 9, 200, 8, 8), (4, 70, 33, 32, 16)])
def test_encoders_match_loop_versions(seed, m, k, br, bc):
    p = synth.random_problem(m, k, 4, 0.08, seed=seed, empty_row_frac=0.15)
    ptr = p.row_ptr.tolist()
    a = oracle.encode_bcsr(m, k, p.row_ptr, p.col_idx, p.vals, br, bc)
    b = _loop_bcsr(m, k, ptr, p.col_idx, p.vals, br, bc)
    assert [x.tolist() for x in a] == [list(x) for x in b]
    a = oracle.encode_wcsr(m, k, p.row_ptr, p.col_idx, p.vals, br, bc)
    b = _loop_wcsr(m, k, ptr, p.col_idx, p.vals, br, bc)
    assert [x.tolist() for x in a] == [list(x) for x in b]


@pytest.mark.parametrize("br,bc", [(16, 16), (64, 64), (16, 8), (32, 32), (8, 8)])
def test_decode_of_encode_is_identity(br, bc):
    p = synth.random_problem(150, 170, 4, 0.05, seed=br + bc, empty_row_frac=0.2)
    rows = p.coo_rows()
    r, c, v = oracle.decode_bcsr(p.m, p.k, *oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals,
                                                               br, bc), br, bc)
    assert np.array_equal(r, rows) and np.array_equal(c, p.col_idx) and np.array_equal(v, p.vals)
    r, c, v = oracle.decode_wcsr(p.m, p.k, *oracle.encode_wcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals,
                                                               br, bc), br)
    assert np.array_equal(r, rows) and np.array_equal(c, p.col_idx) and np.array_equal(v, p.vals)


def test_wcsr_pad_width_is_next_multiple_not_one_more_group():
    # a window with exactly b_col distinct columns is b_col wide (Fig. 2, window 0)
    ptr = np.array([0, 2, 4], np.int32)
    cols = np.array([0, 5, 2, 9], np.int32)
    vals = synth.fp16_bits(np.ones(4))
    wrp, wci, _ = oracle.encode_wcsr(2, 10, ptr, cols, vals, 2, 4)
    assert wrp.tolist() == [0, 4] and wci.tolist() == [0, 2, 5, 9]


# --------------------------------------------------------------------------
# window splitting and tile padding arithmetic
# --------------------------------------------------------------------------

def test_task_rule_hand_example():
    tasks, merges = oracle.wcsr_tasks([0, 8, 8, 40, 48], 16)
    assert tasks.tolist() == [[0, 0, 8, -1], [1, 8, 8, -1], [2, 8, 24, 0], [2, 24, 40, 1], [3, 40, 48, -1]]
    assert merges.tolist() == [[2, 0, 2]]


def test_task_rule_invariants():
    rng = np.random.default_rng(0)
    W = rng.integers(0, 40, size=200) * 8
    wptr = np.concatenate([[0], np.cumsum(W)])
    for T in (32, 64, 96, 1 << 20):
        tasks, merges = oracle.wcsr_tasks(wptr, T)
        # tasks tile every window exactly once, in order, none longer than T
        for w in range(200):
            t = tasks[tasks[:, 0] == w]
            assert t[0, 1] == wptr[w] and t[-1, 2] == wptr[w + 1]
            assert np.array_equal(t[1:, 1], t[:-1, 2])
            assert np.all(t[:, 2] - t[:, 1] <= T)
            assert (len(t) == 1) == (t[0, 3] == -1)
        assert np.array_equal(np.sort(tasks[tasks[:, 3] >= 0, 3]), np.arange(merges[:, 2].sum()))


def test_padding_arithmetic_printed_in_section_iv_c():
    # BN = 496 pads N = 1024 to 1488 (about 45% waste); BN = 352 pads it to 1056 (3%)
    assert oracle.padded_width(1024, 496) == 1488
    assert round((1488 - 1024) / 1024, 2) == 0.45
    assert oracle.padded_width(1024, 352) == 1056
    assert round((1056 - 1024) / 1024, 2) == 0.03
    # 64-wide blocks take 64 / 16 = 4 k16 steps (Section III-A)
    assert 64 // 16 == 4


# --------------------------------------------------------------------------
# reverse Cuthill-McKee (Section IV-A preprocessing)
# --------------------------------------------------------------------------

def _csr_from_edges(n, edges):
    rows = [set() for _ in range(n)]
    for a, b in edges:
        rows[a].add(b)
    row_ptr = np.zeros(n + 1, np.int32)
    cols = []
    for i in range(n):
        c = sorted(rows[i])
        cols += c
        row_ptr[i + 1] = row_ptr[i] + len(c)
    return row_ptr, np.asarray(cols, np.int32)


def _relabelled(n, edges, seed):
    lab = np.random.default_rng(seed).permutation(n)
    return [(int(lab[a]), int(lab[b])) for a, b in edges]


def _bandwidth_after(n, row_ptr, col_idx, perm):
    inv = np.empty(n, np.int64)
    inv[perm] = np.arange(n)
    bw = 0
    for i in range(n):
        for e in range(row_ptr[i], row_ptr[i + 1]):
            bw = max(bw, abs(int(inv[i]) - int(inv[col_idx[e]])))
    return bw


def _is_permutation(perm, n):
    return sorted(perm.tolist()) == list(range(n))


def test_rcm_path_graph_gets_bandwidth_one():
    # a path, relabelled at random and stored one-sided (upper entries only):
    # any level-structure numbering from an end vertex is the path itself
    n = 40
    edges = _relabelled(n, [(i, i + 1) for i in range(n - 1)], seed=1)
    rp, ci = _csr_from_edges(n, edges)
    perm = oracle.rcm_order(n, rp, ci)
    assert _is_permutation(perm, n)
    assert _bandwidth_after(n, rp, ci, perm) == 1


def test_rcm_cycle_gets_bandwidth_two():
    # breadth-first levels of a cycle hold two vertices (one at the ends), and a
    # cycle is not a path: the bandwidth is exactly 2
    n = 33
    edges = _relabelled(n, [(i, (i + 1) % n) for i in range(n)], seed=2)
    edges += [(b, a) for a, b in edges]
    rp, ci = _csr_from_edges(n, edges)
    perm = oracle.rcm_order(n, rp, ci)
    assert _is_permutation(perm, n)
    assert _bandwidth_after(n, rp, ci, perm) == 2


def test_rcm_full_band_is_recovered():
    # full band of half-width b, relabelled: levels from an end vertex hold b
    # consecutive original vertices, so the numbering's bandwidth is <= 2b - 1
    n, b = 300, 7
    edges = [(i, j) for i in range(n) for j in range(i + 1, min(n, i + b + 1))]
    edges = _relabelled(n, edges, seed=3)
    edges += [(q, p) for p, q in edges]
    rp, ci = _csr_from_edges(n, edges)
    perm = oracle.rcm_order(n, rp, ci)
    assert _bandwidth_after(n, rp, ci, perm) <= 2 * b - 1


def test_rcm_hand_examples():
    # orders worked out by hand from the rules in oracle/reorder.py
    # star with centre 3: start at leaf 0, then centre, then leaves by index; reversed
    rp, ci = _csr_from_edges(6, [(3, v) for v in (0, 1, 2, 4, 5)])
    assert oracle.rcm_order(6, rp, ci).tolist() == [5, 4, 2, 1, 3, 0]
    # isolated 2 and 3 first, then component {0, 5} from 0, then path 4-1-6 from 4
    rp, ci = _csr_from_edges(7, [(4, 1), (1, 6), (0, 5)])
    assert oracle.rcm_order(7, rp, ci).tolist() == [6, 1, 4, 5, 0, 3, 2]
    # path 1-2-3-4-5-6 with vertex 0 hanging off 3: the search starts at 0
    # (height 4), moves to 6 (height 5), and 1 is no taller, so numbering starts
    # at 6; at vertex 3 the neighbours go by degree: 0 (1) before 2 (2)
    rp, ci = _csr_from_edges(7, [(1, 2), (2, 3), (3, 4), (4, 5), (5, 6), (0, 3)])
    assert oracle.rcm_order(7, rp, ci).tolist() == [1, 2, 0, 3, 4, 5, 6]


def test_rcm_numbering_is_breadth_first():
    # reversed back, the numbering of each component lists its vertices level by
    # level (distances from the first vertex never decrease), and every vertex
    # after the first is adjacent to an earlier one
    rng = np.random.default_rng(5)
    n = 120
    edges = [(int(a), int(b)) for a, b in rng.integers(0, n, size=(150, 2)) if a != b]
    rp, ci = _csr_from_edges(n, edges)
    adj = oracle.reorder.symmetric_adjacency(n, rp, ci)
    order = oracle.rcm_order(n, rp, ci)[::-1].tolist()
    seen = set()
    i = 0
    while i < n:
        root = order[i]
        dist = oracle.reorder._level_structure(adj, root)
        comp = order[i:i + len(dist)]
        assert set(comp) == set(dist)
        d = [dist[v] for v in comp]
        assert d == sorted(d)
        for v in comp[1:]:
            assert any(w in seen or w == root for w in adj[v] if dist[w] < dist[v])
            seen.add(v)
        seen.add(root)
        i += len(dist)


def test_symmetric_permutation_keeps_the_product():
    # P9: with A' = P A P^T and B' = P B, C' = A' B' is P C (fp64, integer data: exact)
    rng = np.random.default_rng(6)
    n, N = 50, 6
    dense = (rng.random((n, n)) < 0.08) * rng.integers(-3, 4, size=(n, n))
    rows, cols = np.nonzero(dense)
    row_ptr = np.searchsorted(rows, np.arange(n + 1)).astype(np.int32)
    vals = np.asarray([oracle_encode16(float(dense[r, c])) for r, c in zip(rows, cols)], np.uint16)
    B = rng.integers(-3, 4, size=(n, N)).astype(np.float16).view(np.uint16)
    perm = oracle.rcm_order(n, row_ptr, cols.astype(np.int32))
    p_ptr, p_col, p_val = oracle.permute_symmetric(n, row_ptr, cols, vals, perm)
    C, _ = oracle.spmm(n, n, N, rows, cols, vals, B, "fp16")
    prow = np.repeat(np.arange(n), np.diff(p_ptr))
    Cp, _ = oracle.spmm(n, n, N, prow, p_col, p_val, np.ascontiguousarray(B[perm]), "fp16")
    assert np.array_equal(Cp, C[perm])
    # and the permuted pattern is the relabelled one
    D = np.zeros((n, n))
    D[prow, p_col] = oracle.decode16(p_val, "fp16")
    assert np.array_equal(D, dense[np.ix_(perm, perm)])


def oracle_encode16(x: float) -> int:
    return int(np.asarray(x, np.float16).view(np.uint16))


def test_fp8_e4m3_decode_matches_torch_on_all_codes():
    # OCP FP8 E4M3 (the format of gfx950's fp8 MFMA): every one of the 256 codes
    # against torch's float8_e4m3fn, NaN for both NaN codes
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint16)
    ours = oracle.decode16(codes, "fp8")
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref)) and np.isnan(ours).sum() == 2
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert oracle.decode16(np.array([0x7E, 0x01, 0x08, 0xB8]), "fp8").tolist() == [448.0, 2.0 ** -9,
                                                                                    2.0 ** -6, -1.0]


def test_fp8_generator_encoding_matches_torch():
    torch = pytest.importorskip("torch")
    from synth.generators import fp8_e4m3_bits
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (0.002, 0.02, 1.0, 50.0)]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8_e4m3_bits(x), ref.astype(np.uint16))
    # and the oracle's decoder inverts it on its range
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint16)
    assert np.array_equal(fp8_e4m3_bits(oracle.decode16(codes, "fp8")), codes)


# --------------------------------------------------------------------------
# bandwidth and fill ratio: closed forms and independent counts
# --------------------------------------------------------------------------

def _csr_of_pairs(n, pairs):
    pairs = sorted(set(pairs))
    rows = np.array([i for i, _ in pairs], np.int64)
    cols = np.array([j for _, j in pairs], np.int32)
    ptr = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=n))]).astype(np.int32)
    return ptr, cols


def test_bandwidth_closed_forms():
    """max |i - j| (the quantity reverse Cuthill-McKee reduces, Section IV-A)
    on patterns whose value is known without computing it: empty and diagonal
    0, tridiagonal 1, dense n - 1, an arrow (first row and column full) n - 1,
    a band of half-width b exactly b, a single entry (i, j) exactly |i - j|."""
    n = 23
    assert oracle.bandwidth(n, np.zeros(n + 1, np.int32), np.zeros(0, np.int32)) == 0
    assert oracle.bandwidth(n, *_csr_of_pairs(n, [(i, i) for i in range(n)])) == 0
    tri = [(i, j) for i in range(n) for j in (i - 1, i, i + 1) if 0 <= j < n]
    assert oracle.bandwidth(n, *_csr_of_pairs(n, tri)) == 1
    dense = [(i, j) for i in range(n) for j in range(n)]
    assert oracle.bandwidth(n, *_csr_of_pairs(n, dense)) == n - 1
    arrow = [(0, j) for j in range(n)] + [(i, 0) for i in range(n)] + [(i, i) for i in range(n)]
    assert oracle.bandwidth(n, *_csr_of_pairs(n, arrow)) == n - 1
    for b in (2, 5, 9):
        band = [(i, j) for i in range(n) for j in range(max(0, i - b), min(n, i + b + 1))]
        assert oracle.bandwidth(n, *_csr_of_pairs(n, band)) == b
    for i, j in ((0, 17), (17, 0), (22, 3), (11, 11), (21, 22)):
        assert oracle.bandwidth(n, *_csr_of_pairs(n, [(i, j)])) == abs(i - j)


def test_bandwidth_sees_the_largest_offset_anywhere():
    """A tridiagonal pattern with one far entry planted at each position in
    turn (first row, last row, below and above the diagonal): the result is
    that entry's offset, whatever row it sits in."""
    n = 40
    tri = [(i, j) for i in range(n) for j in (i - 1, i, i + 1) if 0 <= j < n]
    for i, j in ((0, 31), (39, 2), (20, 0), (5, 39), (39, 39 - 13)):
        assert oracle.bandwidth(n, *_csr_of_pairs(n, tri + [(i, j)])) == max(1, abs(i - j))


@pytest.mark.parametrize("br,bc", [(4, 4), (16, 8), (64, 64), (3, 5)])
def test_fill_ratio_counts_stored_entries(br, bc):
    """The fill ratio of Section II-C (real nonzeros over stored block
    entries) against a count taken from the encoded blocks themselves: the
    generators never store a zero value, so the nonzero codes in the blocks
    are exactly the real entries and the zero codes the fill."""
    for seed in range(4):
        p = synth.random_problem(97, 130, 8, 0.04 * (seed + 1), seed=seed, empty_row_frac=0.1)
        brp, bci, blocks = oracle.encode_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, br, bc)
        counted = np.count_nonzero(blocks) / blocks.size
        assert oracle.fill_ratio(p.nnz, int(bci.size), br, bc) == pytest.approx(counted, abs=1e-15)


def test_fill_ratio_closed_forms():
    """A full matrix tiled exactly fills every block (1); one entry fills one
    block slot (1 / (b_row * b_col)); the identity of order 64 in 16 x 16
    blocks keeps the 4 diagonal blocks at 16 of 256 entries each (1/16); no
    blocks at all gives 0."""
    assert oracle.fill_ratio(64 * 128, 2 * 2, 32, 64) == 1.0
    assert oracle.fill_ratio(1, 1, 64, 64) == 1 / 4096
    assert oracle.fill_ratio(64, 4, 16, 16) == 1 / 16
    assert oracle.fill_ratio(0, 0, 16, 16) == 0.0

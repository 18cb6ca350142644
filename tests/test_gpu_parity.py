"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Acceptance: |C_gpu - C_ref| <= 2e-3 * sum_k |a_ik||b_kj| elementwise (fp16/bf16
inputs, fp32 accumulation), plus u * |C_ref| for a 16-bit C (one rounding to
nearest: u = 2^-8 bfloat16, 2^-11 binary16); exact equality where the data make
every partial sum exact (small integers).  C is pre-filled with NaN so an
unwritten element fails."""

import os
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ws():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import window_spmm_amd
    return window_spmm_amd


def _device_b(p):
    return torch.from_numpy(p.B.view(np.int16)).cuda()


def run_gpu(ws, p, split_cols=0, A=None, repeats=1):
    _say("gpu case:", p.name, p.fmt, p.m, p.k, p.N, p.b_row, p.b_col, p.ab_dtype, p.c_dtype,
         "split", split_cols)
    if A is None:
        A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                            p.ab_dtype, p.c_dtype, split_cols=split_cols)
    B = _device_b(p)
    outs = []
    for _ in range(repeats):
        C = A.new_c()
        C.fill_(float("nan"))
        A.run(B, C)
        torch.cuda.synchronize()
        outs.append(C.float().cpu().numpy().astype(np.float64))
    return outs if repeats > 1 else outs[0]


def check(p, got, rows=None):
    ref, bound = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, p.ab_dtype,
                             out_rows=rows)
    if rows is not None:
        got = got[rows]
    ok, worst, at = oracle.within_tolerance(got, ref, bound, TOL, out_dtype=p.c_dtype)
    _say("   worst |dC|/Bound = %.3g at %s" % (worst, at))
    assert ok, "parity failed at %s: got %r ref %r bound %r" % (
        at, got[at] if at else None, ref[at] if at else None, bound[at] if at else None)
    return ref


# --------------------------------------------------------------------------
# small cases spanning several tiles and ragged tails
# --------------------------------------------------------------------------

BCSR_CASES = [
    # m, k, N, b_row, b_col, ab, c
    (200, 150, 72, 64, 64, "bf16", "fp32"),
    (256, 256, 64, 16, 16, "fp16", "fp32"),
    (130, 270, 200, 32, 16, "fp16", "bf16"),
    (64, 64, 8, 64, 64, "bf16", "fp16"),
    (1000, 700, 136, 64, 32, "bf16", "bf16"),
    (77, 93, 24, 16, 8, "fp16", "fp32"),
    (300, 500, 520, 64, 64, "bf16", "bf16"),
    (96, 4000, 40, 32, 64, "fp16", "fp32"),
]


@pytest.mark.parametrize("case", BCSR_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bcsr_small(ws, case):
    m, k, N, br, bc, ab, ct = case
    p = synth.block_problem(m, k, N, br, bc, 0.3, seed=m + k, ab_dtype=ab, c_dtype=ct,
                            entry_density=0.7)
    check(p, run_gpu(ws, p))


WCSR_CASES = [
    # m, k, N, b_row, b_col, ab, c, density, split
    (90, 300, 40, 16, 8, "fp16", "fp32", 0.05, 0),
    (1000, 800, 128, 16, 8, "fp16", "fp32", 0.03, 64),
    (517, 1200, 256, 16, 8, "fp16", "fp32", 0.02, 0),
    (300, 300, 32, 16, 8, "bf16", "bf16", 0.05, 32),
    (64, 4000, 128, 32, 16, "fp16", "fp32", 0.05, 96),
    (128, 128, 8, 64, 8, "fp16", "fp16", 0.2, 0),
    (333, 2000, 264, 16, 8, "bf16", "fp32", 0.02, 128),
]


@pytest.mark.parametrize("case", WCSR_CASES, ids=lambda c: "x".join(map(str, c)))
def test_wcsr_small(ws, case):
    m, k, N, br, bc, ab, ct, dens, T = case
    p = synth.random_problem(m, k, N, dens, seed=m + N, ab_dtype=ab, c_dtype=ct, fmt="wcsr",
                             b_row=br, b_col=bc, empty_row_frac=0.1)
    check(p, run_gpu(ws, p, split_cols=T))


@pytest.mark.parametrize("br,bc", [(16, 8), (32, 16), (64, 8)])
def test_wcsr_plan_keeps_its_own_copy_of_the_values(ws, br, bc):
    """A WCSR plan copies the window values into its own fragment-order
    buffer at plan time (widths rounded up to 32 columns with zeros): after
    the caller's value array is overwritten with NaN codes, runs of the plan
    still give the product of the values it was made with, split windows and
    every tile height included."""
    p = synth.random_problem(700, 2500, 136, 0.04, seed=br + bc, ab_dtype="fp16", c_dtype="fp32",
                             fmt="wcsr", b_row=br, b_col=bc, empty_row_frac=0.1)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, split_cols=64)
    assert A.plan.info()["n_merges"] > 0
    A.d_vals.fill_(0x7E00)  # fp16 quiet NaN
    torch.cuda.synchronize()
    check(p, run_gpu(ws, p, A=A))


# --------------------------------------------------------------------------
# exactness, special matrices, edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,br,bc", [("bcsr", 64, 64), ("bcsr", 16, 16), ("wcsr", 16, 8)])
def test_integer_data_is_bit_exact(ws, fmt, br, bc):
    if fmt == "bcsr":
        p = synth.block_problem(320, 300, 136, br, bc, 0.25, seed=7, ab_dtype="fp16",
                                c_dtype="fp32", kind="int", entry_density=0.5)
    else:
        p = synth.random_problem(320, 900, 136, 0.04, seed=7, ab_dtype="fp16", c_dtype="fp32",
                                 kind="int", fmt="wcsr", b_row=br, b_col=bc)
    got = run_gpu(ws, p, split_cols=64 if fmt == "wcsr" else 0)
    ref, _ = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, "fp16")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt,br,bc", [("wcsr", 16, 8), ("bcsr", 64, 64)])
def test_rcm_reordered_product_is_the_permuted_product(ws, fmt, br, bc):
    """P9 through the whole path: with A' = P A P^T (reverse Cuthill-McKee
    order from the library) and B' = P B, the GPU's C' equals P C exactly on
    integer data, and both match the oracle."""
    import dataclasses
    p = synth.random_problem(700, 700, 72, 0.02, seed=23, ab_dtype="fp16", c_dtype="fp32",
                             kind="int", fmt=fmt, b_row=br, b_col=bc)
    perm = ws.rcm_order(p.m, p.row_ptr, p.col_idx)
    rp, ci, v = ws.csr_permute(p.m, p.row_ptr, p.col_idx, p.vals, perm)
    q = dataclasses.replace(p, row_ptr=rp, col_idx=ci, vals=v, B=np.ascontiguousarray(p.B[perm]))
    got = run_gpu(ws, p)
    got_q = run_gpu(ws, q)
    ref, _ = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, "fp16")
    assert np.array_equal(got, ref)
    assert np.array_equal(got_q, ref[perm])


@pytest.mark.parametrize("fmt", ["bcsr", "wcsr"])
def test_identity_gives_b(ws, fmt):
    n, N = 256, 136
    ptr = np.arange(n + 1, dtype=np.int32)
    cols = np.arange(n, dtype=np.int32)
    vals = synth.bf16_bits(np.ones(n))
    B = synth.make_dense_b(np.random.default_rng(3), n, N, "bf16")
    br, bc = (64, 64) if fmt == "bcsr" else (16, 8)
    p = synth.Problem("identity", n, n, N, ptr, cols, vals, B, "bf16", "fp32", fmt, br, bc)
    got = run_gpu(ws, p)
    assert np.array_equal(got, oracle.decode16(B, "bf16").reshape(n, N))


@pytest.mark.parametrize("fmt", ["bcsr", "wcsr"])
def test_empty_matrix_gives_zero(ws, fmt):
    m, k, N = 100, 70, 24
    p = synth.Problem("empty", m, k, N, np.zeros(m + 1, np.int32), np.zeros(0, np.int32),
                      np.zeros(0, np.uint16), synth.make_dense_b(np.random.default_rng(0), k, N, "fp16"),
                      "fp16", "fp32", fmt, 16, 16 if fmt == "bcsr" else 8)
    got = run_gpu(ws, p)
    assert np.array_equal(got, np.zeros((m, N)))


def test_single_entry(ws):
    m, k, N = 64, 64, 128
    ptr = np.zeros(m + 1, np.int32)
    ptr[38:] = 1
    p = synth.Problem("single", m, k, N, ptr, np.array([45], np.int32), synth.fp16_bits(np.array([-1.5])),
                      synth.make_dense_b(np.random.default_rng(1), k, N, "fp16"), "fp16", "fp32",
                      "bcsr", 64, 64)
    got = run_gpu(ws, p)
    b = oracle.decode16(p.B, "fp16").reshape(k, N)
    assert np.array_equal(got[37], -1.5 * b[45])
    assert not np.delete(got, 37, axis=0).any()


def test_empty_rows_and_ragged_m_n(ws):
    # m not a multiple of 64, N with a partial last tile, a third of the rows empty
    p = synth.random_problem(201, 333, 520, 0.05, seed=12, ab_dtype="bf16", c_dtype="bf16",
                             fmt="bcsr", b_row=64, b_col=16, empty_row_frac=0.33)
    got = run_gpu(ws, p)
    ref = check(p, got)
    empty = np.diff(p.row_ptr) == 0
    assert not got[empty].any() and not ref[empty].any()


def test_wcsr_split_invariance_and_determinism(ws):
    p = synth.random_problem(400, 3000, 128, 0.06, seed=5, ab_dtype="fp16", c_dtype="fp32",
                             kind="int", fmt="wcsr", b_row=16, b_col=8)
    ref, _ = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, "fp16")
    for T in (32, 64, 160, 8192):   # 8192: the largest sub-task, no window is cut
        assert np.array_equal(run_gpu(ws, p, split_cols=T), ref), T
    q = synth.random_problem(400, 3000, 128, 0.06, seed=6, ab_dtype="fp16", c_dtype="fp32",
                             fmt="wcsr", b_row=16, b_col=8)
    outs = run_gpu(ws, q, split_cols=64, repeats=20)
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])
    check(q, outs[0])


@pytest.mark.parametrize("ct", ["fp32", "bf16"])
def test_split_merge_across_column_tiles_and_plans(ws, ct):
    """Split row tiles: many split windows, four column tiles (the last one
    ragged), two plans launched alternately and, for each plan, two different B
    matrices in turn (a merge that read partial tiles of an earlier launch
    would show): every launch must give the oracle's result (bit-exact on
    integer data with fp32 C) and the same bits for the same input."""
    kind = "int" if ct == "fp32" else "normal"
    probs = [synth.random_problem(700, 6000, 392, 0.04, seed=31, ab_dtype="fp16", c_dtype=ct,
                                  kind=kind, fmt="wcsr", b_row=16, b_col=8, empty_row_frac=0.1),
             synth.random_problem(260, 2500, 136, 0.08, seed=32, ab_dtype="fp16", c_dtype=ct,
                                  kind=kind, fmt="wcsr", b_row=16, b_col=8)]
    cases = []
    for prob in probs:
        A = ws.DeviceSparse(prob.fmt, prob.m, prob.k, prob.N, prob.row_ptr, prob.col_idx, prob.vals,
                            prob.b_row, prob.b_col, prob.ab_dtype, prob.c_dtype, split_cols=64)
        assert A.plan.info()["n_merges"] > 10, A.plan.info()
        for B in (prob.B, np.ascontiguousarray(prob.B[::-1])):
            ref, bound = oracle.spmm(prob.m, prob.k, prob.N, prob.coo_rows(), prob.col_idx,
                                     prob.vals, B, prob.ab_dtype)
            cases.append((prob, A, torch.from_numpy(B.view(np.int16)).cuda(), ref, bound))
    _say("split merge cases:", [(c[0].name, c[0].N) for c in cases])
    first = {}
    for rep in range(3):
        for i, (prob, A, dB, ref, bound) in enumerate(cases):
            C = A.new_c()
            C.fill_(float("nan"))
            A.run(dB, C)
            torch.cuda.synchronize()
            got = C.float().cpu().numpy().astype(np.float64)
            if kind == "int":
                assert np.array_equal(got, ref), (rep, i)
            else:
                ok, worst, at = oracle.within_tolerance(got, ref, bound, TOL, out_dtype=prob.c_dtype)
                assert ok, (rep, i, at, worst)
            if i in first:
                assert np.array_equal(got, first[i]), (rep, i)
            first.setdefault(i, got)


@pytest.mark.parametrize("source", ["lists", "spread"])
@pytest.mark.parametrize("fmt", ["wcsr", "bcsr"])
def test_work_sources_repeated_launches(ws, fmt, source):
    """Both ways of handing tasks to the work-groups (a list of several tasks
    per persistent work-group, or one task per work-group left to the hardware
    dispatcher) give the oracle's result and the same bits on every one of
    many launches of one plan."""
    opts = {"distribution": 1 if source == "spread" else 0}
    if fmt == "wcsr":
        p = synth.random_problem(1500, 5000, 136, 0.03, seed=21, ab_dtype="fp16", c_dtype="fp32",
                                 fmt="wcsr", b_row=16, b_col=8)
        split = 96
    else:
        p = synth.random_problem(1300, 1100, 72, 0.02, seed=22, ab_dtype="bf16", c_dtype="bf16",
                                 fmt="bcsr", b_row=32, b_col=16)
        split = 0
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, split_cols=split, options=opts)
    outs = run_gpu(ws, p, A=A, repeats=12)
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])
    check(p, outs[0])


def test_bcsr_deterministic(ws):
    p = synth.block_problem(640, 640, 256, 64, 64, 0.3, seed=9, ab_dtype="bf16", c_dtype="fp32")
    outs = run_gpu(ws, p, repeats=10)
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


def test_ld_larger_than_n(ws):
    p = synth.block_problem(128, 128, 64, 64, 64, 0.5, seed=3, ab_dtype="bf16", c_dtype="fp32")
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    Bbig = torch.zeros((p.k, 96), dtype=torch.int16, device="cuda")
    Bbig[:, :64] = _device_b(p)
    Cbig = torch.full((p.m, 80), float("nan"), device="cuda")
    A.run(Bbig[:, :64], Cbig[:, :64])
    torch.cuda.synchronize()
    got = Cbig.cpu().numpy().astype(np.float64)
    assert np.isnan(got[:, 64:]).all()
    check(p, got[:, :64])


@pytest.mark.parametrize("fmt", ["bcsr", "wcsr"])
def test_b_extent_ends_at_last_element(ws, fmt):
    """B with ldb > N in an allocation that ends right after element
    (k - 1) * ldb + N - 1, NaN codes in every row's padding, k and N ragged with
    respect to blocks and column tiles: nothing past N or past the end may reach C."""
    m, k, N, ldb = 700, 650, 200, 264
    if fmt == "bcsr":
        p = synth.block_problem(m, k, N, 64, 64, 0.3, seed=41, ab_dtype="bf16", c_dtype="fp32")
    else:
        p = synth.random_problem(m, k, N, 0.03, seed=42, ab_dtype="fp16", c_dtype="fp32",
                                 fmt="wcsr", b_row=16, b_col=8)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    nan_code = 0x7FC0 if p.ab_dtype == "bf16" else 0x7E00
    flat = np.full((k - 1) * ldb + N, nan_code, dtype=np.uint16)
    for r in range(k):
        flat[r * ldb: r * ldb + N] = p.B[r]
    dev = torch.from_numpy(flat.view(np.int16)).cuda()
    B = torch.as_strided(dev, (k, N), (ldb, 1))
    C = A.new_c()
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    check(p, C.float().cpu().numpy().astype(np.float64))


SWEEP_CASES = [
    # m, k, N, block density, ab, c, ranges per XCD
    (1280, 640, 4104, 0.25, "bf16", "bf16", 1),
    (1280, 640, 4104, 0.25, "bf16", "fp32", 2),
    (700, 600, 8192, 0.3, "fp16", "fp16", 1),
    (640, 512, 4096, 0.95, "bf16", "bf16", 1),
]


@pytest.mark.parametrize("case", SWEEP_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bcsr64_sweep_kernel(ws, case):
    """The A-stationary 64x64 kernel: a ragged last column tile and empty column
    ranges (N not a multiple of 8 tiles), one or two ranges per XCD, padded
    leading dimensions, empty block rows and full (8-block) block rows."""
    m, k, N, dens, ab, ct, H = case
    p = synth.block_problem(m, k, N, 64, 64, dens, seed=m + N + H, ab_dtype=ab, c_dtype=ct)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 2, "ranges_per_xcd": H})
    info = A.plan.info()
    assert info["kernel"] == 2 and info["ranges_per_xcd"] == H
    nblk = np.diff(A.h_ptr)
    assert nblk.max() <= 8
    B = A.device_b(p.B, padded=True)
    C = A.new_c(padded=True)
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    check(p, C.float().cpu().numpy().astype(np.float64))


SWEEP256_CASES = [
    # m, k, N, block density, ab, c, ranges per XCD, kind
    (1280, 640, 4104, 0.25, "bf16", "fp32", 2, "normal"),
    (700, 600, 8192, 0.3, "fp16", "fp16", 1, "normal"),
    (576, 520, 5000, 0.4, "fp16", "fp32", 4, "int"),
    (640, 512, 4096, 0.95, "bf16", "bf16", 1, "normal"),
]


@pytest.mark.parametrize("case", SWEEP256_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bcsr64_sweep_kernel_256_columns(ws, case):
    """The sweep kernel with 4 columns per lane (256-column tiles): ragged m, k
    and N, empty and full block rows, every output type; exact on integer data."""
    m, k, N, dens, ab, ct, H, kind = case
    p = synth.block_problem(m, k, N, 64, 64, dens, seed=m + N + 7 * H, ab_dtype=ab, c_dtype=ct,
                            kind=kind)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype,
                        options={"kernel": 2, "cols_per_lane": 4, "ranges_per_xcd": H})
    info = A.plan.info()
    assert info["kernel"] == 2 and info["cols_per_lane"] == 4 and info["tile_cols"] == 256
    B = A.device_b(p.B, padded=True)
    C = A.new_c(padded=True)
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy().astype(np.float64)
    ref = check(p, got)
    if kind == "int":
        assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def test_config1_full(ws):
    p = synth.config1()
    check(p, run_gpu(ws, p))


def test_config2_full(ws, cfg2):
    check(cfg2, run_gpu(ws, cfg2))


def test_plan_shapes_of_measured_workloads(ws, cfg2):
    """The plan's automatic choices on workloads whose best shape was measured
    (plan sweeps): the 16384^2 WCSR workload takes 8 columns per lane and 4
    reduction waves with no window cut (no merge pass); a small uniform
    population member (50443 rows, about 156 packed columns per window) takes
    one reduction wave."""
    A = ws.DeviceSparse(cfg2.fmt, cfg2.m, cfg2.k, cfg2.N, cfg2.row_ptr, cfg2.col_idx, cfg2.vals,
                        cfg2.b_row, cfg2.b_col, cfg2.ab_dtype, cfg2.c_dtype)
    info = A.plan.info()
    assert (info["cols_per_lane"], info["waves_n"], info["waves_k"], info["n_merges"]) == (8, 1, 4, 0), info
    p = synth.config3_matrix(13, 128, with_b=False)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    info = A.plan.info()
    assert (info["cols_per_lane"], info["waves_k"]) == (8, 1), info


# members up to this many rows are compared with the oracle on every row
CFG3_FULL_ROWS = 60000


def _cfg3_rows(p, seed):
    """Rows of a large population member to compare with the oracle: 512 at
    random, the first and last 16 (ragged last window), and every row of the
    four longest windows (the Zipf tail: these are the windows the plan cuts
    into sub-tasks and merges)."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(p.m, 512, replace=False).tolist())
    rows |= set(range(16)) | set(range(p.m - 16, p.m))
    nw = -(-p.m // p.b_row)
    lens = np.add.reduceat(np.diff(p.row_ptr.astype(np.int64)),
                           np.arange(0, p.m, p.b_row)) if p.m else np.zeros(0)
    for w in np.argsort(-lens)[:4]:
        rows |= set(range(int(w) * p.b_row, min(p.m, (int(w) + 1) * p.b_row)))
    assert nw == lens.size
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("member", range(32))
def test_config3_member_all_n(ws, member):
    """Config 3 run by run: population member `member` at N = 32, 128 and 256
    (the 96 runs of the workload, three per test), through the default plan.
    Members up to 60000 rows are compared with the oracle on every row; larger
    ones on sampled rows that include every row of their longest (split)
    windows; every element of C must have been written (C starts as NaN)."""
    import dataclasses
    p256 = synth.config3_matrix(member, 256)
    for N in (32, 128, 256):
        p = dataclasses.replace(p256, N=N, B=np.ascontiguousarray(p256.B[:, :N]),
                                name="cfg3_m%d_N%d" % (member, N))
        A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row,
                            p.b_col, p.ab_dtype, p.c_dtype)
        _say("   plan", {k: v for k, v in A.plan.info().items()
                         if k in ("tile_cols", "waves_k", "n_tasks", "n_merges")})
        got = run_gpu(ws, p, A=A)
        assert np.isfinite(got).all()
        check(p, got, rows=None if p.m <= CFG3_FULL_ROWS else _cfg3_rows(p, member))
        del A, got


@pytest.mark.parametrize("member,N", [(3, 32), (15, 32), (15, 128), (13, 256)])
def test_config3_members_with_many_merges(ws, member, N):
    """Population members whose Zipf row lengths make a few windows very long:
    the plan cuts them into many 512-column tasks (tens of split windows with up
    to ~18 slots each, so the merge pass runs several rounds per lane group).
    Full parity with the oracle."""
    p = synth.config3_matrix(member, N)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    info = A.plan.info()
    _say("   plan", info)
    assert info["n_merges"] > 0, info
    check(p, run_gpu(ws, p, A=A))


@pytest.mark.parametrize("fmt,N", [("wcsr", 256), ("wcsr", 136), ("bcsr", 264)])
def test_banded_large_b_row_order_wide_tiles(ws, fmt, N):
    """A banded pattern whose B spans several L2s (population member 18: 36674
    rows, band 1 % of n) with few row tiles per resident work-group: the plan
    runs one work-group per row tile in row order with 256-column tiles (N =
    136: one ragged tile; BCSR with 16 x 16 blocks at N = 264: a second, ragged
    column tile and a ragged last block row).  Full parity with the oracle."""
    import dataclasses
    p = synth.config3_matrix(18, 256)
    B = p.B if N <= 256 else np.concatenate([p.B, p.B[:, :N - 256]], axis=1)
    p = dataclasses.replace(p, N=N, B=np.ascontiguousarray(B[:, :N]), fmt=fmt,
                            b_col=16 if fmt == "bcsr" else p.b_col, name="cfg3_m18_%s_N%d" % (fmt, N))
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    info = A.plan.info()
    assert info["tile_cols"] == 256 and info["waves_n"] == 2, info
    check(p, run_gpu(ws, p, A=A))


def _block_rows_sample(p, seed, n_random=48):
    """Random rows plus every row of the first and last block rows."""
    rows = set(np.random.default_rng(seed).choice(p.m, n_random, replace=False).tolist())
    rows |= set(range(min(p.m, p.b_row))) | set(range(max(0, p.m - p.b_row), p.m))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("which", ["gate", "up"])
def test_config4_gate_up_sampled(ws, which):
    """Config 4's 18944 x 3584 weights (gate and up are two seeded draws) at the
    full N = 65536 tokens, the launch configuration the benchmark times: every
    element written, sampled rows (each compared across all 65536 columns, so
    every column tile) against the oracle."""
    p = synth.config4(which)
    got = run_gpu(ws, p)
    assert np.isfinite(got).all()
    check(p, got, rows=_block_rows_sample(p, 1 if which == "gate" else 4))


def test_config4_down_full_n_sampled(ws):
    """Config 4's down weight (3584 x 18944, 30 blocks per block row) at the
    full N = 65536: B is 2.5 GB, so the B offsets reach the top of the 32-bit
    buffer range of the kernels' addressing."""
    p = synth.config4("down")
    got = run_gpu(ws, p)
    assert np.isfinite(got).all()
    check(p, got, rows=_block_rows_sample(p, 2))


def test_config4_down_sampled(ws):
    p = synth.config4("down", N=8192)
    got = run_gpu(ws, p)
    rows = np.random.default_rng(2).choice(p.m, 48, replace=False)
    check(p, got, rows=rows)


RANGE_RULE_CASES = [
    # block density (blocks per block row of 56), N, ranges per XCD the plan takes
    (0.05, 24576, 6),    # 3 blocks, 48 tiles: one-tile ranges, 6 ranges per XCD
    (0.05, 40000, 10),   # 3 blocks, 79 tiles (the last 64 columns wide): one-tile, one empty range
    (0.14, 65536, 2),    # 8 blocks, 128 tiles: two ranges per XCD (8 tiles each)
    (0.02, 65536, 4),    # 1 block, 128 tiles: four ranges per XCD (4 tiles each)
    (0.10, 16384, 1),    # 6 blocks, 32 tiles: one range per XCD (4 tiles each)
]


@pytest.mark.parametrize("case", RANGE_RULE_CASES, ids=lambda c: "d%g-N%d" % c[:2])
def test_sweep_kernel_range_rule_shapes(ws, case):
    """The gate_proj shape (18944 x 3584, 64x64 blocks) at the block counts and
    widths where the sweep kernel's automatic range length changes: the plan
    takes the range count of the rule, and the product (B and C rows allocated
    with the recommended leading dimension, as the benchmark does) matches the
    oracle on sampled rows across all N columns."""
    dens, N, H = case
    p = synth.config4("gate", N=N, density=dens)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    info = A.plan.info()
    assert info["kernel"] == 2 and info["ranges_per_xcd"] == H, info
    _say("gpu case: range rule", dens, N, info)
    B = A.device_b(p.B, padded=True)
    C = A.new_c(padded=True)
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    check(p, got, rows=_block_rows_sample(p, int(N) + 7, n_random=16))


@pytest.mark.parametrize("width", [1, 9])
def test_config5_sampled(ws, width):
    """Config 5 (block-sparse attention probabilities times V): the literal
    pattern (1-block-wide lines) and the variant whose lines are 9 blocks
    wide (about 9 % of causal blocks), on sampled rows."""
    p = synth.config5(width=width)
    got = run_gpu(ws, p)
    assert np.isfinite(got).all()
    rows = np.random.default_rng(3 + width).choice(p.m, 2048, replace=False)
    check(p, got, rows=rows)


WIDE_BCSR_CASES = [
    # m, k, N, b_row, b_col, ab, c: blocks 128 and 256 columns wide, ragged m, k, N
    (200, 700, 72, 16, 128, "fp16", "fp32"),
    (333, 900, 264, 32, 128, "bf16", "bf16"),
    (130, 1000, 136, 64, 128, "bf16", "fp32"),
    (96, 1300, 40, 16, 256, "fp16", "fp16"),
    (250, 777, 200, 32, 256, "bf16", "fp32"),
    (129, 1100, 128, 64, 256, "fp16", "bf16"),
]


@pytest.mark.parametrize("case", WIDE_BCSR_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bcsr_wide_blocks(ws, case):
    """BCSR with 128- and 256-column blocks (the generic kernel's wide-block
    path: several 32-column steps per block, block rows of up to 8192 packed
    columns) on every tile height, ragged m, k and N, all output types."""
    m, k, N, br, bc, ab, ct = case
    p = synth.block_problem(m, k, N, br, bc, 0.4, seed=m + bc, ab_dtype=ab, c_dtype=ct,
                            entry_density=0.5)
    check(p, run_gpu(ws, p))


@pytest.mark.parametrize("br,bc", [(16, 128), (64, 256)])
def test_bcsr_wide_blocks_split_block_row(ws, br, bc):
    """One block row far longer than the others: the plan cuts it into
    sub-tasks whose partial tiles the merge pass adds (n_merges > 0)."""
    import dataclasses
    m, k, N = 8 * br, 40 * bc, 136
    p = synth.block_problem(m, k, N, br, bc, 0.08, seed=br + bc, ab_dtype="bf16",
                            c_dtype="fp32", entry_density=0.3)
    # make block row 3 dense: every entry of its rows present
    dense = synth.block_problem(br, k, N, br, bc, 1.0, seed=5, ab_dtype="bf16", c_dtype="fp32",
                                entry_density=1.0)
    rows = []
    for i in range(m):
        if 3 * br <= i < 4 * br:
            r = i - 3 * br
            rows.append((dense.col_idx[dense.row_ptr[r]:dense.row_ptr[r + 1]],
                         dense.vals[dense.row_ptr[r]:dense.row_ptr[r + 1]]))
        else:
            rows.append((p.col_idx[p.row_ptr[i]:p.row_ptr[i + 1]],
                         p.vals[p.row_ptr[i]:p.row_ptr[i + 1]]))
    ptr = np.concatenate([[0], np.cumsum([len(c) for c, _ in rows])]).astype(np.int32)
    p = dataclasses.replace(p, row_ptr=ptr, col_idx=np.concatenate([c for c, _ in rows]).astype(np.int32),
                            vals=np.concatenate([v for _, v in rows]).astype(np.uint16),
                            name="wide_split_%dx%d" % (br, bc))
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    info = A.plan.info()
    _say("   plan", info)
    assert info["n_merges"] > 0, info
    check(p, run_gpu(ws, p, A=A))


@pytest.mark.parametrize("opts", [{"kernel": 1, "waves_n": 1}, {"kernel": 1, "waves_n": 2},
                                  {"kernel": 1, "waves_n": 4}, {"kernel": 1, "waves_n": 8},
                                  {"kernel": 1, "order": 1}, {"kernel": 0},
                                  {"kernel": 0, "waves_n": 1, "waves_k": 4},
                                  {"kernel": 0, "cols_per_lane": 2, "waves_n": 4}],
                         ids=lambda e: "-".join("%s%s" % (k, v) for k, v in e.items()))
def test_bcsr64_kernel_variants_padded_ld(ws, opts):
    """The 64x64-block kernels (the LDS-shared-A kernel at 2 or 4 waves and in
    launch order, the generic one at several tile shapes, all chosen through
    plan options) on a wide N with padded leading dimensions, a partial last
    column tile, empty block rows and odd block counts."""
    p = synth.block_problem(1280, 640, 1288, 64, 64, 0.25, seed=31, ab_dtype="bf16", c_dtype="bf16")
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options=opts)
    info = A.plan.info()
    for name, value in opts.items():
        if name in ("kernel", "waves_n", "waves_k"):
            assert info[name] == value, (name, info)
        if name == "cols_per_lane":
            assert info["cols_per_lane"] == value
    nblk = np.diff(A.h_ptr)
    assert (nblk == 0).any() and (nblk % 2 == 1).any()
    B = A.device_b(p.B, padded=True)
    C = A.new_c(padded=True)
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    check(p, C.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("kind", ["wcsr16", "bcsr64", "bcsr32"])
def test_every_sweep_candidate_matches_oracle(ws, kind):
    """Every plan option set that `bench.py --sweep` times gives the oracle's
    result (or is refused with UNSUPPORTED before anything runs)."""
    import bench
    if kind == "wcsr16":
        p = synth.random_problem(400, 1500, 136, 0.03, seed=51, ab_dtype="fp16", c_dtype="fp32",
                                 fmt="wcsr", b_row=16, b_col=8)
    elif kind == "bcsr64":
        p = synth.block_problem(330, 520, 4104, 64, 64, 0.3, seed=52, ab_dtype="bf16",
                                c_dtype="bf16")
    else:
        p = synth.block_problem(300, 400, 200, 32, 16, 0.3, seed=53, ab_dtype="fp16",
                                c_dtype="fp32")
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    ref, bound = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, p.ab_dtype)
    B = _device_b(p)
    ran = 0
    for opts in bench.sweep_candidates(p):
        try:
            A.replan(opts)
        except ws.SpmmError as exc:
            assert exc.code == ws.ERR_UNSUPPORTED, (opts, str(exc))
            continue
        _say("   options", opts)
        C = A.new_c()
        C.fill_(float("nan"))
        A.run(B, C)
        torch.cuda.synchronize()
        got = C.float().cpu().numpy().astype(np.float64)
        ok, worst, at = oracle.within_tolerance(got, ref, bound, TOL, out_dtype=p.c_dtype)
        assert ok, (opts, worst, at)
        ran += 1
    assert ran >= 10


COL_MAJOR_CASES = [
    # m, k, N, block density, ab, c, options
    (1000, 520, 1288, 0.3, "bf16", "bf16", {"kernel": 1, "waves_n": 4}),
    (1000, 520, 1288, 0.3, "fp16", "fp32", {"kernel": 1, "waves_n": 2}),
    (520, 640, 200, 0.3, "bf16", "fp32", {"kernel": 1, "waves_n": 1}),
    (1000, 520, 1288, 0.3, "bf16", "bf16", {"kernel": 1, "waves_n": 8}),
    (712, 1096, 4104, 0.45, "fp16", "fp32", {"kernel": 1, "waves_n": 8}),
    (1280, 640, 4104, 0.25, "bf16", "bf16", {"kernel": 2, "ranges_per_xcd": 1}),
    (704, 576, 8200, 0.3, "bf16", "fp16", {"kernel": 2, "ranges_per_xcd": 2}),
    (640, 512, 4096, 0.95, "fp16", "fp32", {"kernel": 2}),
    (1280, 640, 4104, 0.25, "bf16", "bf16", {"kernel": 2, "waves_n": 8, "ranges_per_xcd": 1}),
    (704, 576, 8200, 0.3, "fp16", "fp32", {"kernel": 2, "waves_n": 8}),
    (640, 512, 4096, 0.95, "bf16", "fp16", {"kernel": 2, "waves_n": 8}),
]


@pytest.mark.parametrize("case", COL_MAJOR_CASES, ids=lambda c: "x".join(map(str, c[:6])) + "-k%d" % c[6]["kernel"])
def test_bcsr64_col_major(ws, case):
    """Column-major B and C (B^T: N rows of k, C^T: N rows of m), the layout of
    token-major activations: both 64x64 kernels, N ragged against the column
    tiles, m and k ragged against the blocks, padded leading dimensions with NaN
    codes in B^T's padding; C^T's padding must stay untouched."""
    m, k, N, dens, ab, ct, opts = case
    p = synth.block_problem(m, k, N, 64, 64, dens, seed=m + k + N, ab_dtype=ab, c_dtype=ct)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options=dict(opts, col_major=1))
    info = A.plan.info()
    assert info["col_major"] == 1 and info["kernel"] == opts["kernel"]
    ldb, ldc = k + 24, m + 40
    nan_code = 0x7FC0 if ab == "bf16" else 0x7E00
    bt = np.full((N, ldb), nan_code, dtype=np.uint16)
    bt[:, :k] = p.B.T
    Bt = torch.from_numpy(bt.view(np.int16)).cuda()[:, :k]
    Ct_full = torch.full((N, ldc), float("nan"), device="cuda",
                         dtype={"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[ct])
    A.run(Bt, Ct_full[:, :m])
    torch.cuda.synchronize()
    got = Ct_full.float().cpu().numpy().astype(np.float64)
    assert np.isnan(got[:, m:]).all()
    check(p, np.ascontiguousarray(got[:, :m].T))


@pytest.mark.parametrize("which", ["gate", "down"])
def test_config4_col_major_sampled(ws, which):
    """Config 4's gate and down weights at the full N = 65536 with column-major
    B and C (B^T 65536 x k, C^T 65536 x m, rows allocated with the recommended
    leading dimension), the launch configuration `bench.py --col-major` times:
    every element of C^T written, sampled rows of C (each across all 65536
    columns) against the oracle."""
    p = synth.config4(which)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"col_major": 1})
    info = A.plan.info()
    _say("gpu case: config 4 column-major", which, info)
    assert info["col_major"] == 1 and info["kernel"] == (2 if which == "gate" else 1)
    ldb, ldc = ws.recommended_ld(p.k, 2), ws.recommended_ld(p.m, 2)
    bt = np.zeros((p.N, ldb), dtype=np.uint16)
    bt[:, :p.k] = p.B.T
    Bt = torch.from_numpy(bt.view(np.int16)).cuda()[:, :p.k]
    del bt
    Ct = torch.full((p.N, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :p.m]
    A.run(Bt, Ct)
    torch.cuda.synchronize()
    assert not torch.isnan(Ct).any().item()
    rows = _block_rows_sample(p, 7 if which == "gate" else 8)
    got = np.full((p.m, p.N), np.nan)
    got[rows] = Ct[:, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64).T
    check(p, got, rows=rows)
    del A, Bt, Ct
    torch.cuda.empty_cache()


def test_col_major_rejected_where_unsupported(ws):
    p = synth.block_problem(200, 150, 72, 32, 16, 0.3, seed=1, ab_dtype="bf16", c_dtype="fp32")
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):
        ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"col_major": 1})
    p = synth.block_problem(200, 150, 512, 64, 64, 0.3, seed=2, ab_dtype="bf16", c_dtype="fp32")
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):   # m, k not multiples of 8
        ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"col_major": 1})


# --------------------------------------------------------------------------
# FP8 E4M3 A and B (the sweep kernel)
# --------------------------------------------------------------------------

FP8_CASES = [
    # m, k, N, block density, c, ranges per XCD, kind
    (1280, 640, 4104, 0.25, "bf16", 1, "normal"),
    (700, 600, 8192, 0.3, "fp32", 2, "normal"),
    (640, 512, 4096, 0.95, "fp16", 1, "normal"),
    (576, 520, 5000, 0.4, "fp32", 0, "int"),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8_sweep_kernel(ws, case):
    """FP8 E4M3 A and B, fp32 accumulation: ragged m, k and N, empty and full
    block rows, padded leading dimensions; small-integer data (exact in E4M3,
    every partial sum exact in fp32) must match the oracle bit for bit."""
    m, k, N, dens, ct, H, kind = case
    p = synth.block_problem(m, k, N, 64, 64, dens, seed=m + N + H, ab_dtype="fp8", c_dtype=ct,
                            kind=kind)
    opts = {"ranges_per_xcd": H} if H else None
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options=opts)
    assert A.plan.info()["kernel"] == 2
    assert A.d_vals.dtype == torch.uint8 and A.d_vals.numel() == A.h_vals.size
    B = A.device_b(p.B, padded=True)
    assert B.dtype == torch.uint8 and B.stride(0) == ws.recommended_ld(p.N, 1)
    C = A.new_c(padded=True)
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy().astype(np.float64)
    ref = check(p, got)
    if kind == "int":
        assert np.array_equal(got, ref)


def test_config4_gate_fp8_sampled(ws):
    p = synth.config4("gate", ab_dtype="fp8")
    _say("gpu case:", p.name, p.m, p.k, p.N)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    assert A.plan.info()["kernel"] == 2
    B = A.device_b(p.B)
    C = A.new_c()
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    rows = np.random.default_rng(4).choice(p.m, 48, replace=False)
    check(p, got, rows=rows)


def test_fp8_rejected_where_unsupported(ws):
    def plan(p, options=None, fmt=None):
        return ws.DeviceSparse(fmt or p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row,
                               p.b_col, p.ab_dtype, p.c_dtype, options=options)
    p = synth.block_problem(256, 256, 4096, 64, 64, 0.3, seed=5, ab_dtype="fp8")
    for options in ({"kernel": 1}, {"kernel": 0}, {"col_major": 1}, {"cols_per_lane": 4}):
        with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):
            plan(p, options)
    q = synth.block_problem(256, 256, 4096, 32, 32, 0.3, seed=5, ab_dtype="fp8")
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):
        plan(q)
    q = synth.block_problem(256, 256, 1024, 64, 64, 0.3, seed=5, ab_dtype="fp8")
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):   # N too small for the sweep
        plan(q)
    q = synth.block_problem(128, 1024, 4096, 64, 64, 1.0, seed=5, ab_dtype="fp8")
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):   # 16 blocks in a block row
        plan(q)
    with pytest.raises(ValueError):
        plan(p, fmt="wcsr")


def test_launch_floor_kernel_runs(ws):
    """The empty kernel behind the benchmark's launch floor launches and ends."""
    for _ in range(3):
        ws.launch_floor()
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# kernel 3: BCSR 64 x 64 with A in the registers of a wave pair
# --------------------------------------------------------------------------

def _short_rows_problem(m, k, N, ab, ct, seed, kind="normal", max_blocks=6):
    """64 x 64 BCSR pattern whose block rows hold 0 .. max_blocks blocks (at
    random, so empty rows and odd counts occur), every entry of a kept block
    structural; ragged m and k cut the last block row and block column."""
    from synth.generators import _block_rows_to_csr
    g = np.random.default_rng(seed)
    nbr, nbc = -(-m // 64), -(-k // 64)
    sel = [np.sort(g.choice(nbc, int(g.integers(0, min(max_blocks, nbc) + 1)), replace=False))
           for _ in range(nbr)]
    sel[0] = np.arange(min(max_blocks, nbc))  # one full row
    ptr, cols = _block_rows_to_csr(nbr, 64, 64, m, k, sel)
    enc = synth.bf16_bits if ab == "bf16" else synth.fp16_bits
    if kind == "int":
        v = g.integers(1, 4, cols.size) * g.choice([-1, 1], cols.size)
        b = g.integers(-2, 3, (k, N))
    else:
        v = g.normal(0.0, 1.0, cols.size)
        v[v == 0] = 1.0
        b = g.normal(0.0, 1.0, (k, N))
    return synth.Problem("short_m%d_k%d_N%d_%s_%s_%s" % (m, k, N, ab, ct, kind), m, k, N,
                         ptr.astype(np.int32), cols.astype(np.int32), enc(v.astype(np.float64)),
                         np.ascontiguousarray(enc(b.astype(np.float64))), ab, ct, "bcsr", 64, 64)


PAIR_CASES = [
    # m, k, N, ab, c, ranges per XCD (0: the plan's)
    (1000, 700, 1032, "bf16", "fp32", 0),
    (640, 3584, 2048, "bf16", "bf16", 0),
    (333, 1000, 1160, "fp16", "fp16", 1),
    (700, 450, 4096, "fp16", "fp32", 16),
    (129, 4000, 1024, "bf16", "bf16", 2),
    (64, 64, 1024, "bf16", "fp32", 0),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bcsr64_pair_kernel(ws, case):
    """Kernel 3 on short block rows (0 to 6 blocks, so each wave of the pair
    holds 0 to 3), ragged m, k and N (a partial last strip), every output type,
    one to sixteen column ranges per XCD (sixteen: more ranges than strips, so
    some work-groups have none)."""
    m, k, N, ab, ct, h = case
    p = _short_rows_problem(m, k, N, ab, ct, seed=m + N)
    opts = {"kernel": 3}
    if h:
        opts["ranges_per_xcd"] = h
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options=opts)
    assert A.plan.info()["kernel"] == 3
    check(p, run_gpu(ws, p, A=A))


def test_bcsr64_pair_kernel_integer_exact_padded_ld(ws):
    """Kernel 3 on integer data (every partial sum exact in fp32) with B and C
    rows padded beyond N: bit-equal to the oracle, and two launches agree."""
    p = _short_rows_problem(500, 1300, 1096, "bf16", "fp32", seed=9, kind="int")
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 3})
    ld = p.N + 72
    Bp = torch.full((p.k, ld), -1, dtype=torch.int16, device="cuda")
    Bp[:, :p.N] = torch.from_numpy(p.B.view(np.int16)).cuda()
    Cp = torch.full((p.m, ld), float("nan"), dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        Cp[:, :p.N].fill_(float("nan"))
        A.run(Bp[:, :p.N], Cp[:, :p.N])
        torch.cuda.synchronize()
        outs.append(Cp[:, :p.N].cpu().numpy().astype(np.float64))
    ref, _ = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, p.ab_dtype)
    assert np.array_equal(outs[0], ref) and np.array_equal(outs[1], ref)
    assert torch.isnan(Cp[:, p.N:]).all(), "a store reached the row padding of C"


@pytest.mark.parametrize("which", ["gate", "up"])
def test_config4_pair_kernel_sampled(ws, which):
    """Config 4 gate and up (6 blocks in every block row, N = 65536) through
    kernel 3: every element written, sampled rows against the oracle."""
    p = synth.config4(which)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 3})
    got = run_gpu(ws, p, A=A)
    assert np.isfinite(got).all()
    check(p, got, rows=_block_rows_sample(p, 11 if which == "gate" else 12))


def test_pair_kernel_refused_where_it_cannot_run(ws):
    """Kernel 3 holds at most 6 blocks per block row, 16-bit inputs, row-major
    operands: other problems are refused with UNSUPPORTED."""
    p = _short_rows_problem(256, 1024, 1024, "bf16", "fp32", seed=1, max_blocks=7)
    nb = max(np.diff(ws.csr_to_bcsr(p.m, p.k, p.row_ptr, p.col_idx, p.vals, 64, 64)[0]))
    if nb > 6:
        with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):
            ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, 64, 64,
                            "bf16", "fp32", options={"kernel": 3})
    q = _short_rows_problem(256, 1024, 1024, "bf16", "fp32", seed=2)
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED"):
        ws.DeviceSparse(q.fmt, q.m, q.k, q.N, q.row_ptr, q.col_idx, q.vals, 64, 64, "bf16", "fp32",
                        options={"kernel": 3, "col_major": 1})


# --------------------------------------------------------------------------
# kernel 4: groups of block rows sharing B tiles through an LDS ring
# --------------------------------------------------------------------------

GROUP_CASES = [
    # m, k, N, ab, c, ranges per XCD (0: the plan's)
    (64, 64, 1024, "bf16", "fp32", 0),
    (1000, 700, 1032, "bf16", "fp32", 0),
    (640, 3584, 2048, "bf16", "bf16", 0),
    (333, 1000, 1160, "fp16", "fp16", 1),
    (700, 450, 4096, "fp16", "fp32", 16),
    (129, 4000, 1024, "bf16", "bf16", 2),
    (2000, 1500, 1096, "bf16", "fp32", 4),
]


@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bcsr64_group_kernel(ws, case):
    """Kernel 4 on short block rows (0 to 6 blocks: empty rows, groups whose
    rows share several, one or no block columns, a last group with fewer than
    four rows), ragged m, k and N (a partial last 64-column strip), every output
    type, one to sixteen column ranges per XCD."""
    m, k, N, ab, ct, h = case
    p = _short_rows_problem(m, k, N, ab, ct, seed=m + N + 1)
    opts = {"kernel": 4}
    if h:
        opts["ranges_per_xcd"] = h
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options=opts)
    assert A.plan.info()["kernel"] == 4
    check(p, run_gpu(ws, p, A=A))


def test_bcsr64_group_kernel_integer_exact_repeated(ws):
    """Kernel 4 on integer data: bit-equal to the oracle on three launches in a
    row (the ring's items must reach every consumer intact every time)."""
    p = _short_rows_problem(1280, 2600, 2048, "bf16", "fp32", seed=19, kind="int")
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 4})
    outs = run_gpu(ws, p, A=A, repeats=3)
    ref, _ = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, p.ab_dtype)
    for got in outs:
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("which", ["gate", "up"])
def test_config4_group_kernel_sampled(ws, which):
    """Config 4 gate and up through kernel 4 at N = 65536: every element
    written, sampled rows against the oracle."""
    p = synth.config4(which)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 4})
    got = run_gpu(ws, p, A=A)
    assert np.isfinite(got).all()
    check(p, got, rows=_block_rows_sample(p, 21 if which == "gate" else 22))


# --------------------------------------------------------------------------
# tuned plans (the tile-width measurement of Section IV-C, Fig. 7, made per problem)
# --------------------------------------------------------------------------

def _tuned_case(ws, p, options=None, split_cols=0, rows=None):
    """Tunes a plan on the problem's own B and C, runs it on a NaN-filled C and
    checks the result against the oracle; the options it reports reproduce the
    same configuration through the ordinary plan."""
    _say("gpu case (tuned):", p.name, p.fmt, p.m, p.k, p.N, p.b_row, p.b_col, options)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, split_cols=split_cols, options=options)
    B = _device_b(p)
    C = A.new_c()
    default = A.plan.info()
    chosen = A.tune(B, C, reps=3, options=options)
    info = A.plan.info()
    _say("   default kernel %d tile %d -> tuned %s (kernel %d tile %d, %d timed)" % (
        default["kernel"], default["tile_cols"], chosen, info["kernel"], info["tile_cols"],
        info["tuned"]))
    assert info["tuned"] >= 2
    assert default["tuned"] == 0
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy().astype(np.float64)
    check(p, got, rows=rows)
    if info["split_cols"] in (0, default["split_cols"]):
        A.replan(chosen)
        again = A.plan.info()
        for key in ("kernel", "tile_cols", "waves_n", "waves_k", "cols_per_lane", "ranges_per_xcd"):
            assert again[key] == info[key], key
    return info


def test_tuned_plan_wcsr(ws):
    p = synth.random_problem(1500, 2500, 136, 0.02, seed=61, ab_dtype="fp16", c_dtype="fp32",
                             fmt="wcsr", b_row=16, b_col=8, empty_row_frac=0.1)
    _tuned_case(ws, p)


def test_tuned_plan_wcsr_pinned_fields_stay(ws):
    p = synth.random_problem(700, 900, 72, 0.03, seed=62, ab_dtype="bf16", c_dtype="bf16",
                             fmt="wcsr", b_row=16, b_col=8)
    info = _tuned_case(ws, p, options={"cols_per_lane": 2}, split_cols=64)
    assert info["cols_per_lane"] == 2 and info["split_cols"] == 64


def test_tuned_plan_bcsr64_short_rows(ws):
    p = _short_rows_problem(1000, 1500, 2048, "bf16", "fp32", seed=63)
    _tuned_case(ws, p)


def test_tuned_plan_bcsr_small_blocks(ws):
    p = synth.block_problem(500, 400, 264, 32, 16, 0.3, seed=64, ab_dtype="fp16", c_dtype="bf16",
                            entry_density=0.7)
    _tuned_case(ws, p)


def test_tuned_plan_col_major(ws):
    """A column-major plan tunes among the kernels that take B^T and C^T."""
    p = synth.block_problem(256, 320, 512, 64, 64, 0.3, seed=65, ab_dtype="bf16", c_dtype="fp32",
                            entry_density=0.7)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"col_major": 1})
    Bt = torch.from_numpy(np.ascontiguousarray(p.B.T).view(np.int16)).cuda()
    Ct = torch.empty((p.N, p.m), dtype=torch.float32, device="cuda")
    chosen = A.tune(Bt, Ct, reps=3, options={"col_major": 1})
    info = A.plan.info()
    assert chosen.get("col_major") == 1 and info["col_major"] == 1 and info["kernel"] in (1, 2)
    Ct.fill_(float("nan"))
    A.run(Bt, Ct)
    torch.cuda.synchronize()
    check(p, Ct.T.cpu().numpy().astype(np.float64))


def test_tuned_plan_config3_member(ws):
    """A population member (m = k = 32768 class, banded) at N = 128, tuned."""
    p = synth.config3_matrix(4, 128)
    _tuned_case(ws, p, rows=None if p.m <= CFG3_FULL_ROWS else _cfg3_rows(p, 4))


def test_tuned_plan_refuses_bad_operands(ws):
    p = synth.random_problem(200, 300, 64, 0.05, seed=66, ab_dtype="fp16", c_dtype="fp32",
                             fmt="wcsr", b_row=16, b_col=8)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype)
    B = _device_b(p)
    with pytest.raises(ValueError, match="C has shape"):
        A.tune(B, torch.empty((p.m, p.N + 8), dtype=torch.float32, device="cuda"))
    with pytest.raises(ws.SpmmError):
        A.tune(B, A.new_c(), reps=-1)
    # the object keeps a working plan after a refused tuning
    C = A.new_c()
    A.run(B, C)
    torch.cuda.synchronize()
    check(p, C.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("case", [(1000, 1500, 128, "bf16", "fp32"), (333, 700, 72, "fp16", "bf16"),
                                  (64, 64, 8, "bf16", "fp16"), (520, 4000, 264, "bf16", "fp32")],
                         ids=lambda c: "x".join(map(str, c)))
def test_bcsr64_lds_kernel_one_wave_narrow_n(ws, case):
    """The LDS-shared-A kernel with one wave of 128 columns per work-group (plan
    option waves_n = 1), the only form it takes below N = 256: narrow and ragged
    N (one partial column tile), ragged m and k, every output type."""
    m, k, N, ab, ct = case
    p = synth.block_problem(m, k, N, 64, 64, 0.3, seed=m + N, ab_dtype=ab, c_dtype=ct)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 1, "waves_n": 1})
    info = A.plan.info()
    assert info["kernel"] == 1 and info["waves_n"] == 1 and info["tile_cols"] == 128
    check(p, run_gpu(ws, p, A=A))


def test_bcsr64_lds_kernel_one_wave_below_256(ws):
    """Below N = 256 kernel 1 runs one wave per work-group: the plan's own
    choice for 64x64 blocks from N = 128 (the generic kernel below), the form a
    pinned kernel 1 takes without waves_n, and more waves are refused."""
    p = synth.block_problem(200, 300, 128, 64, 64, 0.3, seed=3, ab_dtype="bf16", c_dtype="fp32")
    for opts in (None, {"kernel": 1}):
        A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                            p.ab_dtype, p.c_dtype, options=opts)
        info = A.plan.info()
        assert info["kernel"] == 1 and info["waves_n"] == 1 and info["tile_cols"] == 128, info
        check(p, run_gpu(ws, p, A=A))
    with pytest.raises(ws.SpmmError) as e:
        ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 1, "waves_n": 2})
    assert e.value.code == ws.ERR_UNSUPPORTED
    q = synth.block_problem(200, 300, 72, 64, 64, 0.3, seed=4, ab_dtype="bf16", c_dtype="fp32")
    A = ws.DeviceSparse(q.fmt, q.m, q.k, q.N, q.row_ptr, q.col_idx, q.vals, q.b_row, q.b_col,
                        q.ab_dtype, q.c_dtype)
    assert A.plan.info()["kernel"] == 0


def test_bcsr64_one_wave_plan_keeps_its_own_copy_of_the_blocks(ws):
    """The one-wave row-major form of kernel 1 reads the plan's fragment-order
    copy of the blocks: after the caller's block array is overwritten with NaN
    codes, runs still give the product of the blocks the plan was made with
    (the automatic plan at N = 128 and kernel 1 pinned to one wave at a wide N
    with a partial last column tile)."""
    for N, opts in ((128, None), (1288, {"kernel": 1, "waves_n": 1})):
        p = synth.block_problem(333, 1000, N, 64, 64, 0.3, seed=N, ab_dtype="bf16", c_dtype="fp32")
        A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                            p.ab_dtype, p.c_dtype, options=opts)
        info = A.plan.info()
        assert info["kernel"] == 1 and info["waves_n"] == 1, info
        A.d_vals.fill_(0x7FC0)  # bf16 quiet NaN
        torch.cuda.synchronize()
        check(p, run_gpu(ws, p, A=A))


def test_config5_generic_kernel_sampled(ws):
    """Config 5 (the block-sparse P*V workload, N = 128, whose automatic plan is
    the one-wave LDS-A kernel) on the generic tile kernel, sampled rows."""
    p = synth.config5()
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, options={"kernel": 0})
    assert A.plan.info()["kernel"] == 0
    got = run_gpu(ws, p, A=A)
    check(p, got, rows=_block_rows_sample(p, 5))



# --------------------------------------------------------------------------
# the largest B the kernels' 32-bit buffer offsets address
# --------------------------------------------------------------------------

# At N = 65536 (leading dimension 66560) the largest k with k * ldb * 2 below
# 2^32 - 256 that is a multiple of 64: B is 4.29 GB.
K_AT_LIMIT = 32256


@pytest.mark.parametrize("fmt,opts", [("bcsr", {}), ("bcsr", {"kernel": 1}), ("bcsr", {"kernel": 0}),
                                      ("bcsr", {"kernel": 3}), ("wcsr", {})],
                         ids=lambda x: x if isinstance(x, str) else ("k%s" % x.get("kernel", "auto")))
def test_b_at_the_32bit_offset_limit(ws, fmt, opts):
    """B of 4.29 GB, the last rows of which sit just below the 2^32 - 256 byte
    limit of the kernels' buffer offsets: A has blocks in the first, a middle and
    the last block columns, so the gathers reach B's last row at every column of
    N = 65536.  The result is compared with the oracle on the B rows A uses."""
    N, k, m = 65536, K_AT_LIMIT, 128
    ldb = ws.recommended_ld(N, 2)
    assert k * ldb * 2 < 2 ** 32 - 256 <= (k + 64) * ldb * 2
    nbc = k // 64
    blocks = [[0, nbc // 2, nbc - 1], [1, nbc - 2, nbc - 1]]
    g = np.random.default_rng(17)
    rows, cols = [], []
    for br, js in enumerate(blocks):
        for r in range(64 * br, 64 * br + 64):
            for J in js:
                rows.append(np.full(64, r))
                cols.append(np.arange(J * 64, J * 64 + 64))
    rows, cols = np.concatenate(rows), np.concatenate(cols)
    row_ptr = np.zeros(m + 1, np.int64)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    v = g.normal(0.0, 1.0, cols.size)
    v[v == 0] = 1.0
    vals = synth.bf16_bits(v)
    _say("gpu case: B at the offset limit", fmt, opts, "k", k, "ldb", ldb)
    # B on the device, drawn there in row chunks
    Bfull = torch.empty((k, ldb), dtype=torch.int16, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    for r0 in range(0, k, 4096):
        r1 = min(k, r0 + 4096)
        Bfull[r0:r1, :N] = torch.randn((r1 - r0, N), generator=gen, device="cuda",
                                        dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    B = Bfull[:, :N]
    b_row, b_col = (64, 64) if fmt == "bcsr" else (16, 8)
    A = ws.DeviceSparse(fmt, m, k, N, row_ptr, cols.astype(np.int32), vals, b_row, b_col, "bf16",
                        "fp32", options=opts or None)
    if opts.get("kernel") is not None:
        assert A.plan.info()["kernel"] == opts["kernel"]
    C = torch.full((m, ws.recommended_ld(N, 4)), float("nan"), dtype=torch.float32, device="cuda")
    A.run(B, C[:, :N])
    torch.cuda.synchronize()
    # the oracle on a compact B holding only the rows A uses
    used = np.unique(cols // 64)
    Bc = B[torch.from_numpy(np.concatenate([np.arange(J * 64, J * 64 + 64) for J in used])).cuda()]
    Bc = Bc.cpu().numpy().view(np.uint16)
    pos = {int(J): i for i, J in enumerate(used)}
    cols_c = np.array([pos[int(c) // 64] * 64 + int(c) % 64 for c in cols], np.int32)
    out_rows = np.array([0, 1, 63, 64, 100, 127])
    ref, bound = oracle.spmm(m, used.size * 64, N, rows.astype(np.int32), cols_c, vals, Bc, "bf16",
                             out_rows=out_rows)
    got = C[:, :N].cpu().numpy().astype(np.float64)[out_rows]
    ok, worst, at = oracle.within_tolerance(got, ref, bound, TOL, out_dtype="fp32")
    _say("   worst |dC|/Bound = %.3g at %s" % (worst, at))
    assert ok, (at, worst)
    assert not np.isnan(C[:, :N].cpu().numpy()).any()
    del Bfull, B, C, A
    torch.cuda.empty_cache()


# Column-major: B^T rows of k = 3584 (7168 bytes, the recommended leading
# dimension), the largest N, a multiple of 8, with N * 7168 below 2^32 - 256:
# B^T is 4.29 GB.
N_CM_AT_LIMIT = 599184


@pytest.mark.parametrize("kernel", [2, 1])
def test_col_major_b_at_the_32bit_offset_limit(ws, kernel):
    """Column-major B^T of 4.29 GB whose last rows sit just below the 2^32 - 256
    byte limit of the kernels' buffer offsets (the whole-line B^T loads address
    rows as row x pitch in 32 bits): A has blocks in the first, a middle and the
    last block columns; sampled columns of C, the last ones among them, are
    compared with the oracle on those columns of B."""
    m, k, N = 128, 3584, N_CM_AT_LIMIT
    ldb = ws.recommended_ld(k, 2)
    assert ldb == k and N * ldb * 2 < 2 ** 32 - 256 <= (N + 8) * ldb * 2
    nbc = k // 64
    blocks = [[0, nbc // 2, nbc - 1], [1, nbc - 2, nbc - 1]]
    rows, cols = [], []
    for br, js in enumerate(blocks):
        for r in range(64 * br, 64 * br + 64):
            for J in js:
                rows.append(np.full(64, r))
                cols.append(np.arange(J * 64, J * 64 + 64))
    rows, cols = np.concatenate(rows), np.concatenate(cols)
    row_ptr = np.zeros(m + 1, np.int64)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    v = np.random.default_rng(23).normal(0.0, 1.0, cols.size)
    v[v == 0] = 1.0
    vals = synth.bf16_bits(v)
    _say("gpu case: column-major B^T at the offset limit, kernel", kernel, "N", N)
    Bt = torch.empty((N, ldb), dtype=torch.int16, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(6)
    for n0 in range(0, N, 65536):
        n1 = min(N, n0 + 65536)
        Bt[n0:n1] = torch.randn((n1 - n0, k), generator=gen, device="cuda",
                                dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    A = ws.DeviceSparse("bcsr", m, k, N, row_ptr, cols.astype(np.int32), vals, 64, 64, "bf16",
                        "fp32", options={"kernel": kernel, "col_major": 1})
    assert A.plan.info()["kernel"] == kernel and A.plan.info()["col_major"] == 1
    Ct = torch.full((N, ws.recommended_ld(m, 4)), float("nan"), dtype=torch.float32,
                    device="cuda")[:, :m]
    A.run(Bt, Ct)
    torch.cuda.synchronize()
    assert not torch.isnan(Ct).any().item()
    sample = np.unique(np.concatenate([np.arange(8), np.arange(N - 72, N),
                                       np.random.default_rng(3).choice(N, 56, replace=False)]))
    Bs = Bt[torch.from_numpy(sample).cuda()].cpu().numpy().view(np.uint16).T.copy()
    ref, bound = oracle.spmm(m, k, sample.size, rows.astype(np.int32), cols.astype(np.int32),
                             vals, Bs, "bf16")
    got = Ct[torch.from_numpy(sample).cuda()].cpu().numpy().astype(np.float64).T
    ok, worst, at = oracle.within_tolerance(got, ref, bound, TOL, out_dtype="fp32")
    _say("   worst |dC|/Bound = %.3g at %s" % (worst, at))
    assert ok, (at, worst)
    del Bt, Ct, A
    torch.cuda.empty_cache()


# The widest N the kernels take: ldb < 2^23 elements (B row numbers and the
# leading dimension share 24-bit multiplies), N = 2^23 - 8.
N_AT_LIMIT = (1 << 23) - 8


@pytest.mark.parametrize("fmt,opts", [("bcsr", {}), ("bcsr", {"kernel": 1}), ("bcsr", {"kernel": 0}),
                                      ("wcsr", {})],
                         ids=lambda x: x if isinstance(x, str) else ("k%s" % x.get("kernel", "auto")))
def test_n_at_the_ldb_limit(ws, fmt, opts):
    """N = 2^23 - 8 columns (B 3.4 GB, C 4.4 GB): thousands of column tiles and
    ranges, the last tile ragged.  The product is separable by columns, so the
    first and the last 8192 columns are compared with the oracle on those
    columns of B."""
    m, k = 130, 200
    N = N_AT_LIMIT
    ldb = ws.recommended_ld(N, 2)
    assert ldb < (1 << 23) and k * ldb * 2 < 2 ** 32 - 256
    b_row, b_col = (64, 64) if fmt == "bcsr" else (16, 8)
    p0 = synth.random_problem(m, k, 8, 0.1, seed=41, ab_dtype="bf16", c_dtype="fp32", fmt=fmt,
                              b_row=b_row, b_col=b_col, empty_row_frac=0.1)
    _say("gpu case: N at the ldb limit", fmt, opts, "N", N)
    Bfull = torch.empty((k, ldb), dtype=torch.int16, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(9)
    for r in range(k):
        Bfull[r, :N] = torch.randn(N, generator=gen, device="cuda", dtype=torch.float32) \
            .to(torch.bfloat16).view(torch.int16)
    B = Bfull[:, :N]
    A = ws.DeviceSparse(fmt, m, k, N, p0.row_ptr, p0.col_idx, p0.vals, b_row, b_col, "bf16", "fp32",
                        options=opts or None)
    if opts.get("kernel") is not None:
        assert A.plan.info()["kernel"] == opts["kernel"]
    C = torch.empty((m, ws.recommended_ld(N, 4)), dtype=torch.float32, device="cuda")[:, :N]
    C.fill_(float("nan"))
    A.run(B, C)
    torch.cuda.synchronize()
    for c0 in (0, N - 8192):
        Bs = B[:, c0:c0 + 8192].contiguous().cpu().numpy().view(np.uint16)
        ref, bound = oracle.spmm(m, k, 8192, p0.coo_rows(), p0.col_idx, p0.vals, Bs, "bf16")
        got = C[:, c0:c0 + 8192].cpu().numpy().astype(np.float64)
        ok, worst, at = oracle.within_tolerance(got, ref, bound, TOL, out_dtype="fp32")
        _say("   columns %d..: worst |dC|/Bound = %.3g at %s" % (c0, worst, at))
        assert ok, (c0, at, worst)
    assert not torch.isnan(C).any().item()
    del Bfull, B, C, A
    torch.cuda.empty_cache()

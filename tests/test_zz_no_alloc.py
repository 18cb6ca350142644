"""The WCSR run that allocates nothing (spmm_wcsr_run_noalloc), through the C
ABI: its output equals spmm_wcsr_run's (same kernels, same fixed merge order,
so bit for bit) and the oracle's, on two calls in a row whose second input is
smaller (fewer split windows: the static scratch keeps the first call's
partial tiles, which the second must not read); plans needing more partial
tiles than the scratch holds are refused with a clear error."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ws():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import window_spmm_amd
    return window_spmm_amd


def _both_runs(ws, p, split_cols):
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, split_cols=split_cols)
    info = A.plan.info()
    _say("case", p.name, "split", split_cols, "merges", info["n_merges"], "slots", info["n_slots"],
         "workspace", A.plan.workspace_bytes)
    B = torch.from_numpy(p.B.view(np.int16)).cuda()
    C_ws = A.new_c()
    C_ws.fill_(float("nan"))
    A.run(B, C_ws)
    C_na = A.new_c()
    C_na.fill_(float("nan"))
    ws.wcsr_run_noalloc(A.plan, B, C_na)
    torch.cuda.synchronize()
    return A, info, C_ws, C_na


def _check_oracle(p, C):
    got = C.float().cpu().numpy().astype(np.float64)
    ref, bound = oracle.spmm(p.m, p.k, p.N, p.coo_rows(), p.col_idx, p.vals, p.B, p.ab_dtype)
    ok, worst, at = oracle.within_tolerance(got, ref, bound, 2e-3, out_dtype=p.c_dtype)
    _say("   worst |dC|/Bound = %.3g" % worst)
    assert ok, "parity failed at %s" % (at,)


def test_noalloc_run_matches_workspace_run_twice_second_smaller(ws):
    first = synth.random_problem(1200, 3000, 256, 0.06, seed=31, ab_dtype="fp16", c_dtype="fp32",
                                 fmt="wcsr", b_row=16, b_col=8)
    second = synth.random_problem(300, 900, 136, 0.05, seed=32, ab_dtype="bf16", c_dtype="bf16",
                                  fmt="wcsr", b_row=16, b_col=8)
    slots = []
    for p, T in ((first, 128), (second, 256)):
        A, info, C_ws, C_na = _both_runs(ws, p, T)
        assert info["n_merges"] > 0, info
        assert 0 < A.plan.workspace_bytes <= ws.NOALLOC_SCRATCH_BYTES
        slots.append(info["n_slots"])
        assert torch.equal(C_ws.view(torch.int32) if C_ws.dtype == torch.float32 else C_ws.view(torch.int16),
                           C_na.view(torch.int32) if C_na.dtype == torch.float32 else C_na.view(torch.int16))
        _check_oracle(p, C_na)
    assert slots[1] < slots[0]


def test_noalloc_run_without_split_windows(ws):
    """A plan with no split window needs no scratch at all."""
    p = synth.random_problem(333, 2000, 264, 0.02, seed=33, ab_dtype="bf16", c_dtype="fp32",
                             fmt="wcsr", b_row=16, b_col=8)
    A, info, C_ws, C_na = _both_runs(ws, p, 8192)  # longer than every window: nothing split
    assert A.plan.workspace_bytes == 0 and info["n_merges"] == 0, info
    assert torch.equal(C_ws, C_na)
    _check_oracle(p, C_na)


def test_noalloc_run_refuses_plans_larger_than_the_scratch(ws):
    """64 windows of about 4000 packed columns cut into 32-column tasks at N = 256
    need about 130 MB of partial tiles, four times the static scratch: the call
    is refused with UNSUPPORTED and names the limit; C is left untouched."""
    p = synth.random_problem(1024, 4096, 256, 0.5, seed=34, ab_dtype="fp16", c_dtype="fp32",
                             fmt="wcsr", b_row=16, b_col=8)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, split_cols=32)
    assert A.plan.workspace_bytes > ws.NOALLOC_SCRATCH_BYTES
    B = torch.from_numpy(p.B.view(np.int16)).cuda()
    C = A.new_c()
    C.fill_(float("nan"))
    with pytest.raises(ws.SpmmError, match="UNSUPPORTED.*static scratch"):
        ws.wcsr_run_noalloc(A.plan, B, C)
    torch.cuda.synchronize()
    assert torch.isnan(C).all()

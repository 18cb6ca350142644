"""SpMM benchmark: effective TFLOP/s of the BCSR / WCSR path on MI355X.

One step = one SpMM C = A*B through the C-ABI on a device-resident synthetic
input (the tile kernel plus, for WCSR windows that were split, the merge
kernel).  Throughput follows the AsyncSparse paper's evaluation (Section IV):
2 * nnz * N / t with nnz the true nonzero count of A; the stored-entry rate
(2 * stored * N / t) is reported next to it.

Default workload: BCSR at the Qwen2.5-7B gate_proj shape (18944 x 3584 bf16
weight, 64 x 64 blocks, 6 of 56 per block row, times 65536 tokens, bf16 out),
the largest of the five workloads; then, as extra keys of the same line, the
WCSR matrix 16384 x 16384 at about 1% density (window 16, column padding 8),
N = 128, fp16 in, fp32 out.  ``--config`` selects another workload (1: small
BCSR, 2: the WCSR matrix alone, 3: one WCSR population member, 5: block-sparse
P*V).  Prints one JSON line.

Timing: `value`, `ms_per_step` and `roofline` use cold-cache time, each launch
preceded by a read of a 1 GiB buffer (more than the 256 MB MALL and the L2s
together), the reads' own time subtracted; warm time (launches back to back,
the paper's protocol) is reported next to it.  ``--warm-only`` skips the cold
pass.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective SpMM TFLOP/s (2·nnz·N) BCSR & WCSR; % of MFMA/HBM roofline"
PEAK_MFMA_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA
PEAK_MFMA_TFLOPS_FP8 = 5000.0  # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
E_C = {"fp32": 4, "bf16": 2, "fp16": 2}
E_AB = {"bf16": 2, "fp16": 2, "fp8": 1}


def make_problem(cfg: int, args):
    import synth
    if cfg == 1:
        return synth.config1(), "cfg1: BCSR 256x256 fp16, 16x16 blocks, 26/256 kept, N=64, fp32 out"
    if cfg == 2:
        return synth.config2(), ("cfg2: WCSR 16384x16384 fp16, lognormal rows (mean ~200), half "
                                 "+-256 band / half uniform, window 16, b_col 8, N=128, fp32 out")
    if cfg == 3:
        p = synth.config3_matrix(args.member, args.n3)
        return p, "cfg3 member %d: WCSR m=k=%d, N=%d, %s" % (
            args.member, p.m, p.N, "banded" if p.meta["banded"] else "uniform")
    if cfg == 4:
        p = synth.config4(args.which, N=args.n4, ab_dtype="fp8" if args.fp8 else "bf16")
        return p, "cfg4 %s: BCSR %dx%d %s, 64x64 blocks, 90%% block sparse, N=%d, bf16 out" % (
            args.which, p.m, p.k, p.ab_dtype, p.N)
    if cfg == 5:
        p = synth.config5(width=args.width)
        return p, "cfg5: BCSR P*V 65536x65536 bf16, 64x64 blocks (diag + 4 vertical + 8 slash%s), " \
                  "N=128, fp32 out" % ("" if args.width == 1 else ", width %d" % args.width)
    raise SystemExit("unknown config %d" % cfg)


def algorithmic(p, A):
    """Flops and the method's compulsory HBM bytes for one SpMM."""
    N = p.N
    stored = A.stored_entries
    if p.fmt == "bcsr":
        nblk = int(A.h_ptr[-1])
        cols = np.unique(A.h_idx)
        brows = int(np.minimum(cols.astype(np.int64) * p.b_col + p.b_col, p.k).sum()
                    - np.minimum(cols.astype(np.int64) * p.b_col, p.k).sum())
        meta = 4 * nblk + 4 * A.h_ptr.size
    else:
        P = A.h_idx.size
        brows = int(np.unique(A.h_idx[A.h_idx >= 0]).size)
        meta = 4 * P + 4 * A.h_ptr.size
    e = E_AB[p.ab_dtype]
    bytes_alg = e * stored + meta + e * N * brows + E_C[p.c_dtype] * p.m * N
    return {"flops_true": 2.0 * p.nnz * N, "flops_stored": 2.0 * stored * N,
            "bytes_alg": float(bytes_alg), "b_rows_referenced": brows}


# the sources of the default plans' kernels (the tile, LDS-A, sweep and merge
# kernels), the headers they include, and the planner that picks their launch
# shapes
KERNEL_SOURCES = [os.path.join(ROOT, "window_spmm_amd", "csrc", f)
                  for f in ("kernels.hip", "kernels.h", "device.h", "api.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def code_only(text: str) -> str:
    """C/C++ source without its comments and blank lines, each line stripped:
    what a traffic record depends on (a comment edit leaves the code, and so
    the counters, as they were).  String and character literals are kept."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return "\n".join(l.strip() for l in "".join(out).splitlines() if l.strip())


def kernel_source_sha256() -> str:
    """One hash over the code (comments and blank lines left out) of the kernel
    and planner sources: a traffic record counts only while it matches."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode("utf-8"))
    return h.hexdigest()


def measured_traffic(workload_key: str):
    """HBM bytes per launch of the dominant kernel from the rocprofv3 counters
    recorded in profiles/traffic.json (FETCH_SIZE and WRITE_SIZE per dispatch,
    each scaled by what the same counter reads for a plain device copy of known
    size), or None when there is no record for this workload or the kernel
    source has changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload_key) if workload_key else None
    if not w or w.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    cp = rec["copy"]
    f_fetch = cp["bytes"] / (cp["fetch_kib"] * 1024.0)
    f_write = cp["bytes"] / (cp["write_kib"] * 1024.0)
    return w["fetch_kib"] * 1024.0 * f_fetch + w["write_kib"] * 1024.0 * f_write


def copy_probe():
    """A plain device-to-device copy of known size (calibrates the FETCH_SIZE and
    WRITE_SIZE counters; run under rocprofv3 --pmc)."""
    import torch
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 5}))


def cpu_baseline(p, budget_s: float):
    """The oracle, as it stands, on all cores of this process, on the same input.
    Repeats the full product until ``budget_s`` has passed (at least once)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    rows = p.coo_rows()
    oracle.spmm(min(p.m, 64), p.k, p.N, rows[rows < 64], p.col_idx[rows < 64], p.vals[rows < 64],
                p.B, p.ab_dtype, nthreads=cores)            # untimed warm-up
    # bounded sample: whole rows from the top of A, at most ~2e9 multiply-adds per pass
    per_row = np.diff(p.row_ptr.astype(np.int64)) * p.N
    cum = np.cumsum(per_row)
    n_rows = int(np.searchsorted(cum, 2e9)) + 1 if cum.size and cum[-1] > 2e9 else p.m
    n_rows = max(1, min(p.m, n_rows))
    sel = rows < n_rows
    r, c, v = rows[sel], p.col_idx[sel], p.vals[sel]
    reps, t_total = 0, 0.0
    while reps == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        oracle.spmm(n_rows, p.k, p.N, r, c, v, p.B, p.ab_dtype, nthreads=cores)
        t_total += time.perf_counter() - t0
        reps += 1
    t = t_total / reps
    # the same sample on one thread, once
    t0 = time.perf_counter()
    oracle.spmm(n_rows, p.k, p.N, r, c, v, p.B, p.ab_dtype, nthreads=1)
    t1 = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": 2.0 * r.size * p.N / t / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "rows 0..%d of the same matrix (%d nonzeros, N=%d), fp64, %d repetition(s), "
                      "%.2f s each" % (n_rows - 1, r.size, p.N, reps, t),
            "one_thread": {"value": 2.0 * r.size * p.N / t1 / 1e12, "seconds": t1},
            "cpu_model": model}


def sweep_candidates(p):
    """Plan options to time: the 64x64 kernels' variants, then the generic
    kernel's tile shapes (columns per lane x waves across N x waves along the
    packed columns) with both ways of handing out tasks."""
    cands = []
    if p.fmt == "bcsr" and p.b_row == 64 and p.b_col == 64:
        cands += [{"kernel": 1, "waves_n": wn, "order": o} for wn in (1, 2, 4, 8) for o in (0, 1)]
        cands += [{"kernel": 2, "ranges_per_xcd": h} for h in (1, 2, 4, 8, 16)]
        cands += [{"kernel": 2, "cols_per_lane": 4, "ranges_per_xcd": h} for h in (1, 2, 4, 8, 16)]
        cands += [{"kernel": 3, "ranges_per_xcd": h} for h in (1, 2, 4, 8, 16, 32)]
        cands += [{"kernel": 4, "ranges_per_xcd": h} for h in (1, 2, 4, 8, 16, 32)]
    for V in (2, 4, 8):
        if V == 8 and p.b_row >= 32:
            continue
        for wn, wk in ((1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (4, 1)):
            for dist in (0, 1):
                cands.append({"kernel": 0, "cols_per_lane": V, "waves_n": wn, "waves_k": wk,
                              "distribution": dist})
    return cands


def run_sweep(p, A, B, C, alg, workload, base=None):
    """Times every candidate plan on the resident input (HIP events on the launch
    stream), checks its C against the default plan's, prints a table and one
    JSON summary line.  The measurement behind choosing a tile width, like the
    paper's sweep over WGMMA_N (Section IV-C, Fig. 7)."""
    import torch
    import window_spmm_amd as ws
    stream = torch.cuda.current_stream()

    def time_plan(n):
        for _ in range(3):
            A.run(B, C, stream)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(n):
            A.run(B, C, stream)
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n * 1e3

    base_us = time_plan(20)
    C_ref = C.float().clone()
    scale = float(C_ref.abs().max()) or 1.0
    rows = [("default", A.plan.info(), base_us, True)]
    for opts in sweep_candidates(p):
        opts = dict(opts, **(base or {}))
        try:
            A.replan(opts)
        except ws.SpmmError as exc:
            rows.append((opts, None, None, str(exc).split(":")[1].strip()))
            continue
        us = time_plan(max(5, min(50, int(2e5 / max(base_us, 1.0)))))
        same = bool(torch.allclose(C.float(), C_ref, rtol=1e-2, atol=1e-3 * scale))
        rows.append((opts, A.plan.info(), us, same))
    A.replan(base)
    # The default plan is timed again after the candidates: the first timing
    # runs on a colder chip than the later ones, the second on a warmer one.
    base_us_last = time_plan(max(5, min(50, int(2e5 / max(base_us, 1.0)))))
    rows.append(("default, timed again last", A.plan.info(), base_us_last, True))
    print("%-64s %6s %10s %9s %7s %s" % ("options", "tile", "us", "TFLOP/s", "frac", "C"))
    best = None
    for opts, info, us, same in rows:
        if info is None:
            print("%-64s %6s %10s %9s %7s %s" % (json.dumps(opts), "-", "-", "-", "-", same))
            continue
        tf = alg["flops_true"] / (us * 1e-6) / 1e12
        peak = PEAK_MFMA_TFLOPS_FP8 if p.ab_dtype == "fp8" else PEAK_MFMA_TFLOPS
        t_roof = max(alg["flops_stored"] / (peak * 1e12), alg["bytes_alg"] / (PEAK_HBM_GBS * 1e9))
        label = (json.dumps(opts) if isinstance(opts, dict) else
                 "%s (kernel %d)" % (opts, info["kernel"]))
        print("%-64s %6d %10.1f %9.1f %7.3f %s" % (label,
                                                  info["tile_cols"], us, tf, t_roof / (us * 1e-6),
                                                  "same" if same is True else "DIFFERS"))
        if same is True and isinstance(opts, dict) and (best is None or us < best[1]):
            best = (opts, us)
    print(json.dumps({"sweep": workload, "default_us": base_us, "default_us_last": base_us_last,
                      "best_options": best[0] if best else None,
                      "best_us": best[1] if best else None}))
    if any(r[3] is False for r in rows):
        raise SystemExit("a candidate plan's C differs from the default plan's")


def run_ffn_table():
    """Kernel-level analog of the paper's gate_proj table (Section IV-D, Table
    III): the 18944 x 3584 gate_proj weight at 80, 90, 95 and 99 % random block
    sparsity (64 x 64 blocks, the same number per block row) times dense
    activations of N = 1K, 4K, 16K and 64K tokens, bf16, against the dense
    product of the same shape through torch.mm (hipBLASLt).  Latency averaged
    over 100 runs after 10 warm-up runs, as in the paper.  At N = 1K each sparse
    result is checked against torch.mm of its densified weight (fp32).  Each
    measurement is preceded by at least 100 ms of the same launches (at least
    10), so that it starts at the clock the load holds rather than at an idle
    one; sparse cases before the dense one."""
    import torch
    import synth
    import window_spmm_amd as ws
    dev = torch.device("cuda:0")
    m, k = 18944, 3584
    sparsities = (0.80, 0.90, 0.95, 0.99)

    def timed(fn, warm=10, n=100, warm_ms=100.0):
        torch.cuda.synchronize()
        t0, done = time.perf_counter(), 0
        while done < warm or (time.perf_counter() - t0) * 1e3 < warm_ms:
            fn()
            done += 1
            if done % 10 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n

    rows = []
    for N in (1024, 4096, 16384, 65536):
        g = torch.Generator(device=dev)
        g.manual_seed(N)
        Bf = torch.randn((k, N), generator=g, device=dev).to(torch.bfloat16)
        ld = ws.recommended_ld(N, 2)
        Bp = torch.empty((k, ld), dtype=torch.int16, device=dev)
        Bp[:, :N] = Bf.view(torch.int16)
        B = Bp[:, :N]
        row = {"N": N}
        for sp in sparsities:
            p = synth.config4("gate", N=N, with_b=False, density=1.0 - sp)
            A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row,
                                p.b_col, p.ab_dtype, p.c_dtype, device=dev)
            C = A.new_c(dev, padded=True)
            t_sp = timed(lambda: A.run(B, C))
            check = None
            if N == 1024:
                W = torch.zeros((m, k), dtype=torch.float32)
                rr = torch.from_numpy(np.repeat(np.arange(m), np.diff(p.row_ptr)))
                W[rr, torch.from_numpy(p.col_idx.astype(np.int64))] = \
                    torch.from_numpy(p.vals.view(np.int16).copy()).view(torch.bfloat16).float()
                ref = torch.mm(W.to(dev), Bf.float())
                err = (C.float() - ref).abs().max().item()
                check = err <= 2e-2 * max(1.0, ref.abs().max().item())
                del W, ref
            row["s%d" % round(sp * 100)] = {"ms": t_sp,
                                             "kernel": A.plan.info()["kernel"],
                                             "blocks_per_row": p.meta["blocks_per_row"],
                                             "checked": check}
            del A, C
        Wd = (torch.randn((m, k), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        Cd = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        t_dense = timed(lambda: torch.mm(Wd, Bf, out=Cd))
        del Wd
        row["dense_ms"] = t_dense
        for sp in sparsities:
            row["s%d" % round(sp * 100)]["speedup"] = t_dense / row["s%d" % round(sp * 100)]["ms"]
        rows.append(row)
        print("N=%6d dense %.3f ms | " % (N, t_dense) + " | ".join(
            "%d%%: %.3f ms (%.2fx, k%d)" % (round(sp * 100), row["s%d" % round(sp * 100)]["ms"],
                                             row["s%d" % round(sp * 100)]["speedup"],
                                             row["s%d" % round(sp * 100)]["kernel"])
            for sp in sparsities), flush=True)
        del Bf, Bp, B, Cd
    print(json.dumps({"ffn_gate_table": rows}))
    if any(r[k_]["checked"] is False for r in rows for k_ in r if k_.startswith("s")):
        raise SystemExit("a sparse result disagrees with torch.mm of its densified weight")


def time_calls(launch, steps, warmup):
    """Time (s) of one call of `launch(stream)` on the current stream: after
    warm-up, one HIP event pair around `steps` back-to-back calls, divided by
    `steps`.  Returns (per-call event time, per-call wall time)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        launch(stream)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s.record(stream)
    for _ in range(steps):
        launch(stream)
    e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / 1e3 / steps, wall / steps


def time_runs(A, B, C, steps, warmup):
    """time_calls for one SpMM through the plan of A."""
    return time_calls(lambda st: A.run(B, C, st), steps, warmup)


def timed_pair(A, B, C, steps, warmup, cold=True):
    """Warm and cold per-launch time (s) of one SpMM.

    Warm: after `warmup` launches, one HIP event pair on the launch stream
    around `steps` back-to-back launches.  Cold: `steps` steps of (sum of a
    1 GiB buffer, launch): the sum reads more than the MALL and every L2 hold,
    so each launch starts with its inputs in HBM only, and it leaves no dirty
    lines whose write-back would overlap the launch (a fill would); the region
    of `steps` sums alone is timed the same way and subtracted.  Every region
    is bracketed by torch.cuda.synchronize() on both sides.  Returns (warm,
    cold or None, the regions' raw times in ms)."""
    import torch
    t_warm, wall_warm = time_runs(A, B, C, steps, warmup)
    region = {"warm_ms": t_warm * steps * 1e3, "warm_wall_ms": wall_warm * steps * 1e3}
    if not cold:
        return t_warm, None, region
    flush = torch.ones(1 << 28, dtype=torch.float32, device=C.device)
    sink = torch.empty((), dtype=torch.float32, device=C.device)
    t_pair, _ = time_calls(lambda st: (torch.sum(flush, dim=0, out=sink), A.run(B, C, st)), steps, 2)
    t_read, _ = time_calls(lambda st: torch.sum(flush, dim=0, out=sink), steps, 2)
    del flush, sink
    region.update({"flush_and_run_ms": t_pair * steps * 1e3, "flush_only_ms": t_read * steps * 1e3})
    return t_warm, max(t_pair - t_read, 1e-9), region


def roofline_of(p, alg, t, info, key):
    """The roofline record of one launch time t (s): the bound (MFMA or HBM,
    whichever takes longer at its published peak), achieved rate, fraction,
    and the HBM traffic the counters recorded for this workload."""
    peak_mfma = PEAK_MFMA_TFLOPS_FP8 if p.ab_dtype == "fp8" else PEAK_MFMA_TFLOPS
    t_roof_mfma = alg["flops_stored"] / (peak_mfma * 1e12)
    t_roof_hbm = alg["bytes_alg"] / (PEAK_HBM_GBS * 1e9)
    if t_roof_hbm >= t_roof_mfma:
        roof = {"bound": "hbm", "achieved": alg["bytes_alg"] / t / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": alg["flops_stored"] / t / 1e12,
                "peak": peak_mfma, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(key)
    roof["traffic_unit"] = "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["kernel_us"] = t * 1e6
    roof["kernels"] = KERNEL_NAMES.get(info["kernel"], "spmm_tile_kernel") + \
        (" + wcsr_merge_kernel" if info["n_merges"] else "")
    return roof


KERNEL_NAMES = {0: "spmm_tile_kernel", 1: "bcsr64_lds_kernel", 2: "bcsr64_sweep_kernel",
                3: "bcsr64_pair_kernel", 4: "bcsr64_group_kernel"}


def wcsr_extra(args, dev):
    """The WCSR half of the default line: the 16384^2 matrix at about 1%
    density, window 16, N = 128, timed warm and cold like the main workload."""
    import torch
    import window_spmm_amd as ws
    print("bench: WCSR workload (config 2)", file=sys.stderr, flush=True)
    p, workload = make_problem(2, args)
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, device=dev)
    B = A.device_b(p.B, dev, padded=True)
    C = A.new_c(dev, padded=True)
    alg = algorithmic(p, A)
    info = A.plan.info()
    t_warm, t_cold, region = timed_pair(A, B, C, max(args.steps, 20), args.warmup,
                                        not args.warm_only)
    t = t_cold if t_cold is not None else t_warm
    t_roof = roofline_time(p, alg)
    out = {"workload": workload, "timing": "cold" if t_cold is not None else "warm",
           "tflops_true": alg["flops_true"] / t / 1e12,
           "tflops_stored": alg["flops_stored"] / t / 1e12,
           "roofline_fraction": t_roof / t, "t_roof_us": t_roof * 1e6,
           "warm_us": t_warm * 1e6, "roofline_fraction_warm": t_roof / t_warm,
           "bytes_alg": alg["bytes_alg"], "nnz": p.nnz, "stored_entries": A.stored_entries,
           "roofline": roofline_of(p, alg, t, info, "config2"),
           "plan": {k: info[k] for k in ("kernel", "tile_cols", "waves_n", "waves_k",
                                         "cols_per_lane", "split_cols", "n_tasks", "n_merges")},
           "timed_regions": region}
    if t_cold is not None:
        out["cold_us"] = t_cold * 1e6
    del A, B, C
    torch.cuda.empty_cache()
    return out


def measured_peaks():
    """What this GPU reaches on plain dense work, timed like a run, next to the
    published peaks the roofline uses: a 1 GiB device-to-device copy (HBM read
    plus write) and an 8192^3 bf16 GEMM through torch.mm (hipBLASLt)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    t_copy, _ = time_calls(lambda st: b.copy_(a), 10, 3)
    del a, b
    m = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    x = torch.randn((m, m), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.randn((m, m), generator=g, device="cuda").to(torch.bfloat16)
    z = torch.empty_like(x)
    t_mm, _ = time_calls(lambda st: torch.mm(x, y, out=z), 10, 3)
    del x, y, z
    return {"hbm_copy_GBs": 2.0 * n * 4 / t_copy / 1e9,
            "dense_bf16_gemm_TFLOPs": 2.0 * m ** 3 / t_mm / 1e12,
            "how": "1 GiB fp32 device copy (read + write bytes); torch.mm 8192^3 bf16; "
                   "one event pair around 10 launches after 3 warm-up launches"}


def launch_floor(steps=100, warmup=10):
    """Per-launch time (s) of the library's empty kernel, timed like a run."""
    import window_spmm_amd as ws
    return time_calls(lambda st: ws.launch_floor(st), steps, warmup)[0]


def roofline_time(p, alg):
    """t_roof = max(stored flops / MFMA peak, algorithmic bytes / HBM peak) in s."""
    peak = PEAK_MFMA_TFLOPS_FP8 if p.ab_dtype == "fp8" else PEAK_MFMA_TFLOPS
    return max(alg["flops_stored"] / (peak * 1e12), alg["bytes_alg"] / (PEAK_HBM_GBS * 1e9))


def tuned_pair(A, B, C, p, alg, args):
    """A tuned plan (spmm_wcsr_plan_tuned on the run's own B and C) beside the
    default plan: three rounds that time the default and the tuned plan in
    turn, like the default timing, and the median of each."""
    import torch
    import window_spmm_amd as ws
    tplan, chosen = ws.wcsr_plan_tuned(p.m, p.k, p.N, p.b_row, p.b_col, A.h_ptr, A.d_idx,
                                       A.d_vals, B, C, p.ab_dtype, p.c_dtype)
    nb = tplan.workspace_bytes
    tws = torch.empty(max(1, (nb + 3) // 4), dtype=torch.float32, device=C.device) if nb else None
    t_def, t_tun = [], []
    for _ in range(3):
        t_def.append(time_runs(A, B, C, args.steps, args.warmup)[0])
        t_tun.append(time_calls(lambda st: ws.wcsr_run(tplan, B, C, tws, st), args.steps,
                                args.warmup)[0])
    td, tt = sorted(t_def)[1], sorted(t_tun)[1]
    info = tplan.info()
    tplan.destroy()
    return {"us": tt * 1e6, "us_default": td * 1e6, "tflops_true": alg["flops_true"] / tt / 1e12,
            "frac": roofline_time(p, alg) / tt, "frac_default": roofline_time(p, alg) / td,
            "options": chosen, "kernel": info["kernel"], "tile_cols": info["tile_cols"],
            "split_cols": info["split_cols"], "timed": info["tuned"]}


def run_population(args):
    """Config 3 as the workload defines it: every matrix of the seeded WCSR
    population (32 matrices, m = k from 8K to 512K, banded and uniform, Zipf
    row lengths) at N = 32, 128 and 256, timed like the paper's runs (warm-up,
    then HIP events around each launch), with geometric means of the effective
    TFLOP/s (2*nnz*N/t) and of the roofline fractions over the 96 runs and per
    N.  Stands in for the paper's SuiteSparse collection, which is not used."""
    import dataclasses
    import torch
    import synth
    import window_spmm_amd as ws
    dev = torch.device("cuda:0")
    specs = synth.config3_specs()
    members = range(len(specs))
    if args.members:
        lo, _, hi = args.members.partition("-")
        members = range(int(lo), int(hi or lo) + 1)
    floor = launch_floor()
    print("bench: launch floor %.2f us" % (floor * 1e6), file=sys.stderr, flush=True)
    runs = []
    for j in members:
        print("bench: population member %d (m=%d, mean row %.1f, %s)" % (
            j, specs[j][0], specs[j][1], "banded" if specs[j][2] else "uniform"),
            file=sys.stderr, flush=True)
        p256 = synth.config3_matrix(j, 256)
        for N in (32, 128, 256):
            p = dataclasses.replace(p256, N=N, B=np.ascontiguousarray(p256.B[:, :N]),
                                    name="cfg3_m%d_N%d" % (j, N))
            A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row,
                                p.b_col, p.ab_dtype, p.c_dtype, device=dev)
            B = A.device_b(p.B, dev, padded=True)
            C = A.new_c(dev, padded=True)
            t, _ = time_runs(A, B, C, args.steps, args.warmup)
            alg = algorithmic(p, A)
            info = A.plan.info()
            tuned = None
            if args.tuned:
                tuned = tuned_pair(A, B, C, p, alg, args)
            r = {"member": j, "m": p.m, "nnz": p.nnz, "banded": bool(p.meta["banded"]), "N": N,
                 "us": t * 1e6, "tflops_true": alg["flops_true"] / t / 1e12,
                 "frac": roofline_time(p, alg) / t, "t_roof_us": roofline_time(p, alg) * 1e6,
                 "frac_with_floor": min(1.0, (roofline_time(p, alg) + floor) / t),
                 "fill": p.nnz / A.stored_entries, "n_tasks": info["n_tasks"],
                 "n_merges": info["n_merges"]}
            if tuned is not None:
                r["tuned"] = tuned
            runs.append(r)
            print("bench:   N=%3d %9.1f us  %7.2f TFLOP/s  frac %.3f  (t_roof %.1f us, fill %.3f, "
                  "%d tasks, %d merges)" % (N, r["us"], r["tflops_true"], r["frac"], r["t_roof_us"],
                                            r["fill"], r["n_tasks"], r["n_merges"]),
                  file=sys.stderr, flush=True)
            if tuned is not None:
                print("bench:          tuned %9.1f us (default %.1f us, interleaved)  frac %.3f  "
                      "%s split %d" % (tuned["us"], tuned["us_default"], tuned["frac"],
                                       json.dumps(tuned["options"]), tuned["split_cols"]),
                      file=sys.stderr, flush=True)
            del A, B, C
        del p256
        torch.cuda.empty_cache()

    def gm(xs):
        return float(np.exp(np.mean(np.log(xs)))) if xs else None

    out = {"population": "cfg3: 32 seeded WCSR matrices x N in {32, 128, 256}, window 16, "
                          "b_col 8, fp16 in, fp32 out",
           "runs": len(runs), "steps": args.steps, "warmup": args.warmup,
           "geomean_tflops_true": gm([r["tflops_true"] for r in runs]),
           "geomean_frac": gm([r["frac"] for r in runs]),
           "launch_floor_us": floor * 1e6,
           "geomean_frac_with_floor": gm([r["frac_with_floor"] for r in runs]),
           "per_N": {N: {"geomean_tflops_true": gm([r["tflops_true"] for r in runs if r["N"] == N]),
                         "geomean_frac": gm([r["frac"] for r in runs if r["N"] == N])}
                     for N in (32, 128, 256)},
           "detail": runs}
    if args.tuned:
        out["tuned"] = {
            "how": "spmm_wcsr_plan_tuned per run (candidates timed on the run's own B and C); "
                   "then three rounds timing the default and the tuned plan in turn, medians",
            "geomean_tflops_true": gm([r["tuned"]["tflops_true"] for r in runs]),
            "geomean_frac": gm([r["tuned"]["frac"] for r in runs]),
            "geomean_frac_default_interleaved": gm([r["tuned"]["frac_default"] for r in runs]),
            "geomean_speedup": gm([r["tuned"]["us_default"] / r["tuned"]["us"] for r in runs]),
            "per_N": {N: {"geomean_frac": gm([r["tuned"]["frac"] for r in runs if r["N"] == N]),
                          "geomean_frac_default_interleaved":
                              gm([r["tuned"]["frac_default"] for r in runs if r["N"] == N])}
                      for N in (32, 128, 256)}}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--which", default="gate", help="config 4 weight: gate, up or down")
    ap.add_argument("--member", type=int, default=0, help="config 3 matrix index")
    ap.add_argument("--population", action="store_true",
                    help="config 3: every matrix of the population at N = 32, 128, 256, geo-means")
    ap.add_argument("--members", default="", help="with --population: a range of members, e.g. 0-7")
    ap.add_argument("--n3", type=int, default=128, help="config 3 N")
    ap.add_argument("--n4", type=int, default=65536, help="config 4 N (tokens)")
    ap.add_argument("--width", type=int, default=1, help="config 5 line width in blocks")
    ap.add_argument("--split", type=int, default=0, help="WCSR sub-task size (0 = plan's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--tuned", action="store_true",
                    help="time a tuned plan (spmm_*_plan_tuned) instead of the default one; "
                         "with --population: tune each run's plan and report it beside the "
                         "default plan")
    ap.add_argument("--warm-only", action="store_true",
                    help="no cold-cache pass: value and roofline from warm launches")
    ap.add_argument("--no-peaks", action="store_true",
                    help="leave out the measured copy and GEMM peaks (for profiled runs)")
    ap.add_argument("--no-wcsr", action="store_true",
                    help="default workload: leave out the WCSR (config 2) extra keys")
    ap.add_argument("--no-pad", action="store_true", help="B and C with leading dimension N")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the kernel / tile-shape options on this workload instead")
    ap.add_argument("--ffn-table", action="store_true",
                    help="gate_proj latency at 80-99%% block sparsity x N = 1K..64K against "
                         "dense torch.mm (the paper's Table III, kernel level)")
    ap.add_argument("--fp8", action="store_true",
                    help="config 4 with FP8 E4M3 weights and activations")
    ap.add_argument("--options", default="",
                    help="plan options to pin, as JSON (e.g. '{\"kernel\": 3, \"ranges_per_xcd\": 8}')")
    ap.add_argument("--col-major", action="store_true",
                    help="BCSR 64x64: B and C column-major (B^T: N x k, C^T: N x m), the "
                         "token-major activation layout")
    args = ap.parse_args()
    if args.fp8 and args.config != 4:
        raise SystemExit("--fp8 applies to config 4")

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.ffn_table:
        run_ffn_table()
        return
    if args.population:
        run_population(args)
        return

    import torch
    import window_spmm_amd as ws

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    print("bench: generating config %d" % args.config, file=sys.stderr, flush=True)
    p, workload = make_problem(args.config, args)
    print("bench: building format and plan", file=sys.stderr, flush=True)
    opts = json.loads(args.options) if args.options else {}
    if args.col_major:
        opts["col_major"] = 1
    A = ws.DeviceSparse(p.fmt, p.m, p.k, p.N, p.row_ptr, p.col_idx, p.vals, p.b_row, p.b_col,
                        p.ab_dtype, p.c_dtype, device=dev, split_cols=args.split,
                        options=opts or None)
    info = A.plan.info()
    if args.col_major:
        # B^T (N x k) and C^T (N x m), rows padded like the row-major operands
        ldb = p.k if args.no_pad else ws.recommended_ld(p.k, 2)
        ldc = p.m if args.no_pad else ws.recommended_ld(p.m, E_C[p.c_dtype])
        bt = np.zeros((p.N, ldb), dtype=np.uint16)
        bt[:, :p.k] = p.B.T
        B = torch.from_numpy(bt.view(np.int16)).to(dev)[:, :p.k]
        del bt
        cdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[p.c_dtype]
        C = torch.empty((p.N, ldc), dtype=cdt, device=dev)[:, :p.m]
        workload += " [column-major B^T, C^T]"
    else:
        # B and C rows padded to the library's recommended leading dimension (only
        # differs from N when the row pitch is a multiple of 4 KiB, e.g. N = 65536)
        B = A.device_b(p.B, dev, padded=not args.no_pad)
        C = A.new_c(dev, padded=not args.no_pad)
    alg = algorithmic(p, A)
    if args.sweep:
        run_sweep(p, A, B, C, alg, workload, {"col_major": 1} if args.col_major else None)
        return
    tuned_opts = None
    if args.tuned:
        # the plan chosen by timing (spmm_*_plan_tuned on this B and C) instead of
        # the plan's rules; the options it returns are reported in config
        print("bench: tuning the plan", file=sys.stderr, flush=True)
        tuned_opts = A.tune(B, C, options=opts or None)
        info = A.plan.info()

    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t_warm, t_cold, region = timed_pair(A, B, C, args.steps, args.warmup, not args.warm_only)
    t_kernel = t_cold if t_cold is not None else t_warm

    key = "config%d" % args.config + ("_" + args.which if args.config == 4 else "") + \
          ("_m%d_n%d" % (args.member, args.n3) if args.config == 3 else "") + \
          ("_w%d" % args.width if args.config == 5 and args.width != 1 else "") + \
          ("_colmajor" if args.col_major else "") + ("_fp8" if args.fp8 else "")
    if opts or args.tuned or args.n4 != 65536:
        key = None   # the traffic records hold the default plans of the named workloads
    roof = roofline_of(p, alg, t_kernel, info, key)
    peak_mfma = PEAK_MFMA_TFLOPS_FP8 if p.ab_dtype == "fp8" else PEAK_MFMA_TFLOPS
    t_roof_mfma = alg["flops_stored"] / (peak_mfma * 1e12)
    t_roof_hbm = alg["bytes_alg"] / (PEAK_HBM_GBS * 1e9)
    ms_step = t_kernel * 1e3

    value = alg["flops_true"] / t_kernel / 1e12
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.ab_dtype,
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": workload, "format": p.fmt, "m": p.m, "k": p.k, "N": p.N,
                   "options": opts,
                   "tuned": None if tuned_opts is None else {"options": tuned_opts,
                                                             "configurations_timed": info["tuned"]},
                   "ldb": int(B.stride(0)), "ldc": int(C.stride(0)),
                   "b_row": p.b_row, "b_col": p.b_col, "nnz": p.nnz,
                   "stored_entries": A.stored_entries, "c_dtype": p.c_dtype,
                   "plan": {k: info[k] for k in ("kernel", "tile_cols", "waves_n", "waves_k", "cols_per_lane",
                                                 "ranges_per_xcd", "split_cols", "n_tasks", "n_merges")}},
        "timing": "cold" if t_cold is not None else "warm",
        "tflops_true": value,
        "tflops_stored": alg["flops_stored"] / t_kernel / 1e12,
        "roofline_fraction": max(t_roof_mfma, t_roof_hbm) / t_kernel,
        "t_roof_us": max(t_roof_mfma, t_roof_hbm) * 1e6,
        "bytes_alg": alg["bytes_alg"],
        "warm_us": t_warm * 1e6,
        "roofline_fraction_warm": max(t_roof_mfma, t_roof_hbm) / t_warm,
        "tflops_true_warm": alg["flops_true"] / t_warm / 1e12,
        "roofline": roof,
        "timed_regions": region,
    }
    if t_cold is not None:
        out["cold_us"] = t_cold * 1e6
        out["roofline_fraction_cold"] = max(t_roof_mfma, t_roof_hbm) / t_cold
    floor = launch_floor()
    out["launch_floor_us"] = floor * 1e6
    out["roofline_fraction_with_floor"] = min(1.0, (max(t_roof_mfma, t_roof_hbm) + floor) / t_kernel)
    if not args.no_cpu:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    default_line = args.config == 4 and args.which == "gate" and not (args.fp8 or args.col_major) \
        and args.n4 == 65536
    if default_line and not args.no_wcsr:
        del A, B, C
        torch.cuda.empty_cache()
        out["wcsr_cfg2"] = wcsr_extra(args, dev)
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Seeded generators for the five SpMM workloads and for small fuzz cases.

Every array is a pure function of (config id, matrix id, stream, seed):
``numpy.random.Generator(PCG64(SeedSequence([config, matrix, stream, seed])))``
with stream 0 = sparsity pattern, 1 = values of A, 2 = dense operand B.

Output is a sparse pattern in CSR order (rows ascending, columns ascending and
unique inside a row) together with 16-bit value bits (IEEE fp16 or bfloat16)
and a dense row-major B as 16-bit bits.  The CSR arrays are also valid COO
triplets (row of entry t = the row whose range holds t).

The workload shapes follow the AsyncSparse paper (Liu, Pu, Zhang, 2026):
the SuiteSparse-like populations of Section IV-A are replaced by seeded
scattered/banded patterns, the Qwen2.5-7B FFN shapes come from Section IV-D
(Table III) and the block-sparse attention-probability product uses a
vertical + slash block pattern in the style of the sparse attention used in
Section IV-D.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Problem", "rng_for", "fp16_bits", "bf16_bits", "make_dense_b",
    "config1", "config2", "config3_specs", "config3_matrix", "config4",
    "config5", "random_problem", "block_problem",
]


# --------------------------------------------------------------------------
# basic helpers: PRNG streams and 16-bit conversion of draws
# --------------------------------------------------------------------------

def rng_for(config_id: int, matrix_id: int, stream: int, seed: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([int(config_id), int(matrix_id), int(stream), int(seed)])))


def fp16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 bits of ``x`` (numpy's round-to-nearest-even)."""
    return np.asarray(x).astype(np.float16).view(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bits of ``x``: fp32 (RNE) first, then RNE on the fp32 bits."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes of ``x`` (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits, subnormals down to 2^-9, no infinities), round to nearest
    even, magnitudes past 448 saturated to 448; returned as uint16 (0..255)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    sign = np.signbit(np.asarray(x, dtype=np.float64)).astype(np.uint16) << 7
    out = np.zeros(a.shape, dtype=np.uint16)
    sub = a < 2.0 ** -6
    # subnormal: m * 2^-9 with m = 0..8 (m = 8 is the code of 2^-6, the smallest normal)
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.uint16)
    mant, ex = np.frexp(a[~sub])            # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1             # a = (2 mant) * 2^e
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)   # 3 fraction bits, 0..8
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    big = (e > 8) | ((e == 8) & (q > 6))
    e = np.where(big, 8, e)
    q = np.where(big, 6, q)
    out[~sub] = (((e + 7) << 3) | q).astype(np.uint16)
    return out | sign


def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return fp16_bits(x)
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "fp8":
        return fp8_e4m3_bits(x)
    raise ValueError(dtype)


def _nonzero_values(rng: np.random.Generator, n: int, dtype: str, draw) -> np.ndarray:
    """``n`` value bits from ``draw(rng, size)``; draws that round to +-0 are redrawn,
    so every structural entry holds a nonzero value."""
    bits = _bits(draw(rng, n), dtype)
    mag = 0x7F if dtype == "fp8" else 0x7FFF
    while True:
        z = np.flatnonzero((bits & mag) == 0)
        if z.size == 0:
            return bits
        bits[z] = _bits(draw(rng, z.size), dtype)


def make_dense_b(rng: np.random.Generator, k: int, n: int, dtype: str,
                 chunk: int = 1 << 24) -> np.ndarray:
    """Dense row-major ``k x n`` operand with N(0, 1) entries, as 16-bit bits.
    Drawn in fixed-size chunks (fp32 normal draws) so that big operands never need
    a float64 copy; the chunking is part of the recipe."""
    total = int(k) * int(n)
    out = np.empty(total, dtype=np.uint16)
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        out[s:e] = _bits(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(k, n)


# --------------------------------------------------------------------------
# distinct sampling per row (vectorised rejection)
# --------------------------------------------------------------------------

def _sample_rows(rng, size, count):
    """For every row r draw ``count[r]`` distinct integers in ``[0, size[r])``.

    Returns ``vals`` sorted by (row, value); row r owns
    ``vals[ptr[r]:ptr[r+1]]`` with ``ptr = concat([0], cumsum(count))``.
    Rows asking for more than half of their range draw the complement instead.
    """
    size = np.asarray(size, dtype=np.int64)
    count = np.asarray(count, dtype=np.int64)
    if np.any(count > size) or np.any(count < 0):
        raise ValueError("count out of range")
    n = size.size
    comp = 2 * count > size
    draw = np.where(comp, size - count, count)
    rows = np.repeat(np.arange(n, dtype=np.int64), draw)
    vals = np.minimum((rng.random(rows.size) * size[rows]).astype(np.int64), size[rows] - 1)
    big = np.int64(1) << np.int64(32)
    while True:
        key = rows * big + vals
        order = np.argsort(key, kind="stable")
        ks = key[order]
        dup = np.zeros(rows.size, dtype=bool)
        dup[order[1:][ks[1:] == ks[:-1]]] = True
        nd = int(dup.sum())
        if nd == 0:
            break
        vals[dup] = np.minimum((rng.random(nd) * size[rows[dup]]).astype(np.int64),
                               size[rows[dup]] - 1)
    picked = vals[order]
    if not comp.any():
        return picked
    # complement rows: keep everything in [0, size) that was not drawn
    prow = rows[order]
    cidx = np.flatnonzero(comp)
    csize = size[cidx]
    cstart = np.concatenate([[0], np.cumsum(csize)])
    keep = np.ones(int(cstart[-1]), dtype=bool)
    local = np.full(n, -1, dtype=np.int64)
    local[cidx] = np.arange(cidx.size)
    sel = comp[prow]
    keep[cstart[local[prow[sel]]] + picked[sel]] = False
    crow = np.repeat(cidx, csize)
    cval = np.arange(int(cstart[-1]), dtype=np.int64) - np.repeat(cstart[:-1], csize)
    crow, cval = crow[keep], cval[keep]
    allrow = np.concatenate([prow[~sel], crow])
    allval = np.concatenate([picked[~sel], cval])
    order = np.lexsort((allval, allrow))
    return allval[order]


def _extend_rows(rng, base_ptr, base_vals, need, k):
    """Add ``need[r]`` new distinct columns from ``[0, k)`` to every row, avoiding
    the row's existing columns.  Returns (ptr, vals) sorted within rows."""
    n = need.size
    base_rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(base_ptr))
    new_rows = np.repeat(np.arange(n, dtype=np.int64), need)
    new_vals = np.minimum((rng.random(new_rows.size) * k).astype(np.int64), k - 1)
    big = np.int64(1) << np.int64(32)
    while True:
        rows = np.concatenate([base_rows, new_rows])
        vals = np.concatenate([base_vals.astype(np.int64), new_vals])
        isnew = np.concatenate([np.zeros(base_rows.size, bool), np.ones(new_rows.size, bool)])
        pos = np.arange(rows.size)
        # sort by (row, value, existing-first, arrival order)
        order = np.lexsort((pos, isnew, vals, rows))
        key = (rows * big + vals)[order]
        dupsorted = np.zeros(rows.size, dtype=bool)
        dupsorted[1:] = key[1:] == key[:-1]
        dup = np.zeros(rows.size, dtype=bool)
        dup[order[dupsorted]] = True
        ndup = dup[base_rows.size:]
        nd = int(ndup.sum())
        if nd == 0:
            break
        new_vals[ndup] = np.minimum((rng.random(nd) * k).astype(np.int64), k - 1)
    order = np.lexsort((vals, rows))
    counts = np.diff(base_ptr) + need
    ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return ptr, vals[order]


# --------------------------------------------------------------------------
# problem container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Problem:
    """One SpMM instance: C[m x N] = A[m x k] * B[k x N]."""
    name: str
    m: int
    k: int
    N: int
    row_ptr: np.ndarray      # int32[m+1]  (CSR, columns sorted and unique per row)
    col_idx: np.ndarray      # int32[nnz]
    vals: np.ndarray         # uint16[nnz] value bits in ab_dtype
    B: np.ndarray            # uint16[k, N] row-major bits in ab_dtype
    ab_dtype: str            # "fp16" | "bf16"
    c_dtype: str             # "fp32" | "bf16" | "fp16"
    fmt: str                 # "bcsr" | "wcsr"
    b_row: int
    b_col: int
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.col_idx.size)

    def coo_rows(self) -> np.ndarray:
        return np.repeat(np.arange(self.m, dtype=np.int32), np.diff(self.row_ptr))


def _finish(name, m, k, N, ptr, cols, vals, B, ab, c, fmt, br, bc, **meta) -> Problem:
    ptr = np.asarray(ptr, dtype=np.int64)
    if ptr[-1] >= 2 ** 31:
        raise ValueError("nnz does not fit int32")
    return Problem(name, int(m), int(k), int(N), ptr.astype(np.int32),
                   np.asarray(cols, dtype=np.int32), np.asarray(vals, dtype=np.uint16),
                   B, ab, c, fmt, int(br), int(bc), dict(meta))


def _block_rows_to_csr(nbr, br, bc, m, k, block_cols_per_row):
    """Expand kept blocks (list of sorted block-column arrays per block row) into a
    CSR pattern where every entry of a kept block is structural."""
    counts = np.zeros(m, dtype=np.int64)
    pieces = []
    for I in range(nbr):
        J = np.asarray(block_cols_per_row[I], dtype=np.int64)
        cols = (J[:, None] * bc + np.arange(bc)[None, :]).reshape(-1)
        cols = cols[cols < k]
        r0, r1 = I * br, min(m, (I + 1) * br)
        counts[r0:r1] = cols.size
        pieces.append(np.tile(cols, r1 - r0))
    ptr = np.concatenate([[0], np.cumsum(counts)])
    return ptr, (np.concatenate(pieces) if pieces else np.zeros(0, np.int64))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def config1(seed: int = 0) -> Problem:
    """256x256 fp16, 16x16 blocks, 26 of the 256 block positions kept uniformly;
    every entry of a kept block is structural; values N(0,1); B 256x64 N(0,1);
    fp32 output."""
    m = k = 256
    br = bc = 16
    N = 64
    r0 = rng_for(1, 0, 0, seed)
    pos = np.sort(r0.choice(256, size=26, replace=False))
    per_row = [[] for _ in range(16)]
    for p in pos:
        per_row[p // 16].append(p % 16)
    ptr, cols = _block_rows_to_csr(16, br, bc, m, k, [sorted(x) for x in per_row])
    vals = _nonzero_values(rng_for(1, 0, 1, seed), cols.size, "fp16",
                           lambda g, n: g.standard_normal(n))
    B = make_dense_b(rng_for(1, 0, 2, seed), k, N, "fp16")
    return _finish("cfg1_bcsr_256", m, k, N, ptr, cols, vals, B, "fp16", "fp32", "bcsr", br, bc,
                   kept_blocks=26)


def config2(seed: int = 0) -> Problem:
    """16384x16384 fp16 at about 1% density: row lengths lognormal(ln 120, 1)
    rounded and clipped to [1, 4096]; half of each row (floor) inside a +-256
    band around the diagonal, the rest uniform over all columns; values U(-1,1);
    window height 16, column padding 8; B 16384x128 N(0,1); fp32 output."""
    m = k = 16384
    N = 128
    g = rng_for(2, 0, 0, seed)
    nnz_r = np.clip(np.rint(g.lognormal(math.log(120.0), 1.0, size=m)), 1, 4096).astype(np.int64)
    i = np.arange(m, dtype=np.int64)
    lo = np.maximum(0, i - 256)
    hi = np.minimum(k - 1, i + 256)
    bsize = hi - lo + 1
    n_band = np.minimum(nnz_r // 2, bsize)
    band = _sample_rows(g, bsize, n_band) + np.repeat(lo, n_band)
    bptr = np.concatenate([[0], np.cumsum(n_band)])
    ptr, cols = _extend_rows(g, bptr, band, nnz_r - n_band, k)
    vals = _nonzero_values(rng_for(2, 0, 1, seed), cols.size, "fp16",
                           lambda r, n: r.uniform(-1.0, 1.0, n))
    B = make_dense_b(rng_for(2, 0, 2, seed), k, N, "fp16")
    return _finish("cfg2_wcsr_16k", m, k, N, ptr, cols, vals, B, "fp16", "fp32", "wcsr", 16, 8)


def _cfg3_dims(g):
    m = int(round(math.exp(g.uniform(math.log(8192), math.log(524288)))))
    mu = float(math.exp(g.uniform(math.log(4), math.log(256))))
    return m, mu


def config3_specs(seed: int = 0, count: int = 32):
    """(m, target mean nnz per row, banded?) for each matrix of the population."""
    return [_cfg3_dims(rng_for(3, j, 0, seed)) + (j % 2 == 0,) for j in range(count)]


def _zipf_row_lengths(g, m, mu, cap):
    """Per-row lengths: Zipf(1.5) draws x, scaled by s and clipped to [1, cap];
    s is found by bisection (log scale) so that the mean length is closest to mu."""
    x = g.zipf(1.5, size=m).astype(np.float64)
    capf = cap.astype(np.float64)

    def mean_for(s):
        return float(np.clip(np.rint(s * x), 1.0, capf).mean())

    lo, hi = 1e-6, 1.0
    while mean_for(hi) < mu and hi < 1e12:
        hi *= 2.0
    for _ in range(100):
        mid = math.sqrt(lo * hi)
        if mean_for(mid) < mu:
            lo = mid
        else:
            hi = mid
    s = lo if abs(mean_for(lo) - mu) <= abs(mean_for(hi) - mu) else hi
    return np.clip(np.rint(s * x), 1.0, capf).astype(np.int64), s


def config3_matrix(j: int, N: int, seed: int = 0, with_b: bool = True) -> Problem:
    """Matrix ``j`` of the population: m = k log-uniform in [8192, 524288], mean row
    length log-uniform in [4, 256], Zipf(1.5) row lengths rescaled to that mean;
    even j banded (|i-col| <= floor(0.01 m)), odd j uniform; values U(-1,1) fp16;
    B m x N N(0,1) (the same B rows for every N, truncated); fp32 output."""
    g = rng_for(3, j, 0, seed)
    m, mu = _cfg3_dims(g)
    banded = j % 2 == 0
    k = m
    i = np.arange(m, dtype=np.int64)
    if banded:
        bw = int(math.floor(0.01 * m))
        lo = np.maximum(0, i - bw)
        hi = np.minimum(k - 1, i + bw)
        cap = hi - lo + 1
    else:
        lo = np.zeros(m, dtype=np.int64)
        cap = np.full(m, k, dtype=np.int64)
    nnz_r, s = _zipf_row_lengths(g, m, mu, cap)
    cols = _sample_rows(g, cap, nnz_r) + np.repeat(lo, nnz_r)
    ptr = np.concatenate([[0], np.cumsum(nnz_r)])
    vals = _nonzero_values(rng_for(3, j, 1, seed), cols.size, "fp16",
                           lambda r, n: r.uniform(-1.0, 1.0, n))
    if with_b:
        B = make_dense_b(rng_for(3, j, 2, seed), k, 256, "fp16")
        B = np.ascontiguousarray(B[:, :N])
    else:
        B = np.zeros((0, N), np.uint16)
    return _finish(f"cfg3_wcsr_m{j}_N{N}", m, k, N, ptr, cols, vals, B, "fp16", "fp32", "wcsr",
                   16, 8, matrix=j, banded=banded, target_mean=mu, scale=s)


_CFG4_SHAPES = {"gate": (18944, 3584, 0), "up": (18944, 3584, 1), "down": (3584, 18944, 2)}


def config4(which: str = "gate", N: int = 65536, seed: int = 0, with_b: bool = True,
            density: float = 0.1, ab_dtype: str = "bf16") -> Problem:
    """Qwen2.5-7B MLP weight shapes (gate/up 18944x3584, down 3584x18944), bf16
    N(0, 0.02), 64x64 blocks, each block row keeps round(density * block
    columns) blocks (at least one) chosen uniformly without replacement;
    activations K x N bf16 N(0,1); bf16 output.  density = 0.1 is the 90 %
    block sparsity of the workload; other values serve the sparsity sweep.
    ab_dtype = "fp8": the same pattern with FP8 E4M3 weights and activations,
    weights drawn N(0, 1) (as if pre-multiplied by a per-tensor scale of 50,
    which keeps them clear of the E4M3 subnormals)."""
    m, k, mid = _CFG4_SHAPES[which]
    br = bc = 64
    nbr, nbc = m // br, k // bc
    keep = max(1, int(round(density * nbc)))
    g = rng_for(4, mid, 0, seed)
    sel = _sample_rows(g, np.full(nbr, nbc), np.full(nbr, keep)).reshape(nbr, keep)
    ptr, cols = _block_rows_to_csr(nbr, br, bc, m, k, list(sel))
    if ab_dtype not in ("bf16", "fp8"):
        raise ValueError(ab_dtype)
    sd = 0.02 if ab_dtype == "bf16" else 1.0
    vals = _nonzero_values(rng_for(4, mid, 1, seed), cols.size, ab_dtype,
                           lambda r, n: r.normal(0.0, sd, n))
    B = make_dense_b(rng_for(4, mid, 2, seed), k, N, ab_dtype) if with_b else np.zeros((0, N), np.uint16)
    return _finish(f"cfg4_bcsr_{which}" + ("_fp8" if ab_dtype == "fp8" else ""), m, k, N, ptr,
                   cols, vals, B, ab_dtype, "bf16", "bcsr", br, bc, which=which,
                   blocks_per_row=keep)


def config5(seed: int = 0, width: int = 1, N: int = 128, with_b: bool = True) -> Problem:
    """Block-sparse attention probabilities times V: 65536x65536 bf16, 64x64 blocks
    on the causal block diagonal, 4 seeded vertical block columns (blocks (r, c)
    with r >= c) and 8 seeded slash diagonals (blocks (r, r - d)); ``width``
    widens every vertical/slash line to that many blocks.  Inside kept blocks the
    token-level causal mask (col <= row) applies; values U(0,1) divided by their
    row's fp64 sum, then rounded to bf16; V 65536x128 bf16 N(0,1); fp32 output."""
    m = k = 65536
    br = bc = 64
    nb = m // br
    g = rng_for(5, 0, 0, seed)
    vcols = np.sort(g.choice(nb, size=4, replace=False))
    slash = np.sort(g.choice(np.arange(1, nb), size=8, replace=False))
    vset = set()
    for c in vcols:
        vset.update(range(int(c), min(nb, int(c) + width)))
    dset = set()
    for d in slash:
        dset.update(range(int(d), min(nb, int(d) + width)))
    varr = np.array(sorted(vset), dtype=np.int64)
    darr = np.array(sorted(dset), dtype=np.int64)
    counts = np.zeros(m, dtype=np.int64)
    pieces = []
    nblocks = 0
    for r in range(nb):
        blk = set(varr[varr < r].tolist()) | set((r - darr[darr <= r]).tolist())
        off = np.array(sorted(blk), dtype=np.int64)
        nblocks += off.size + 1
        base = (off[:, None] * bc + np.arange(bc)[None, :]).reshape(-1)
        for t in range(br):
            i = r * br + t
            row = np.concatenate([base, r * bc + np.arange(t + 1)])
            counts[i] = row.size
            pieces.append(row)
    ptr = np.concatenate([[0], np.cumsum(counts)])
    cols = np.concatenate(pieces)
    gv = rng_for(5, 0, 1, seed)
    u = gv.random(cols.size)
    while True:
        z = np.flatnonzero(u == 0.0)
        if z.size == 0:
            break
        u[z] = gv.random(z.size)
    rows = np.repeat(np.arange(m), counts)
    sums = np.bincount(rows, weights=u, minlength=m)
    vals = bf16_bits((u / sums[rows]).astype(np.float32))
    if np.any((vals & 0x7FFF) == 0):
        raise RuntimeError("normalised value rounded to zero")
    B = make_dense_b(rng_for(5, 0, 2, seed), k, N, "bf16") if with_b else np.zeros((0, N), np.uint16)
    return _finish(f"cfg5_bcsr_pv{'' if width == 1 else f'_w{width}'}", m, k, N, ptr, cols, vals, B,
                   "bf16", "fp32", "bcsr", br, bc, vertical=vcols.tolist(), slash=slash.tolist(),
                   width=width, kept_blocks=nblocks)


# --------------------------------------------------------------------------
# small fuzz / special inputs
# --------------------------------------------------------------------------

_VALUE_DRAWS = {
    "normal": lambda r, n: r.standard_normal(n),
    "uniform": lambda r, n: r.uniform(-1.0, 1.0, n),
    # small nonzero integers: products and short sums stay exact in fp32
    "int": lambda r, n: r.choice(np.array([-4, -3, -2, -1, 1, 2, 3, 4], dtype=np.float64), n),
    "positive": lambda r, n: r.uniform(0.0, 1.0, n) + 1e-3,
}


def _b_draw(g, k, N, ab, kind):
    if kind == "int":
        x = g.integers(-8, 9, size=(k, N)).astype(np.float64)
        return _bits(x, ab).reshape(k, N)
    if kind == "positive":
        return _bits(g.uniform(0.0, 1.0, size=(k, N)), ab).reshape(k, N)
    return make_dense_b(g, k, N, ab)


def random_problem(m: int, k: int, N: int, density: float, seed: int = 0, ab_dtype: str = "fp16",
                   c_dtype: str = "fp32", kind: str = "normal", fmt: str = "wcsr", b_row: int = 16,
                   b_col: int = 8, empty_row_frac: float = 0.0, max_row: Optional[int] = None) -> Problem:
    """Scattered pattern: row lengths Binomial(k, density), columns uniform and
    distinct; a fraction of rows forced empty; values from ``kind``."""
    g = rng_for(100, seed, 0, 0)
    cnt = g.binomial(k, density, size=m).astype(np.int64) if k > 0 else np.zeros(m, np.int64)
    if max_row is not None:
        cnt = np.minimum(cnt, max_row)
    if empty_row_frac > 0:
        cnt[g.random(m) < empty_row_frac] = 0
    cnt = np.minimum(cnt, k)
    cols = _sample_rows(g, np.full(m, k), cnt) if m > 0 else np.zeros(0, np.int64)
    ptr = np.concatenate([[0], np.cumsum(cnt)])
    vals = _nonzero_values(rng_for(100, seed, 1, 0), cols.size, ab_dtype, _VALUE_DRAWS[kind])
    B = _b_draw(rng_for(100, seed, 2, 0), k, N, ab_dtype, kind)
    return _finish(f"rand_m{m}_k{k}_N{N}_s{seed}", m, k, N, ptr, cols, vals, B, ab_dtype, c_dtype,
                   fmt, b_row, b_col)


def block_problem(m: int, k: int, N: int, b_row: int, b_col: int, block_density: float,
                  seed: int = 0, ab_dtype: str = "bf16", c_dtype: str = "fp32", kind: str = "normal",
                  entry_density: float = 1.0) -> Problem:
    """Block-clustered pattern: each b_row x b_col block position kept with
    probability ``block_density``; inside kept blocks each entry kept with
    probability ``entry_density`` (1.0 = all structural)."""
    g = rng_for(101, seed, 0, 0)
    nbr = -(-m // b_row)
    nbc = -(-k // b_col)
    keep = g.random((nbr, nbc)) < block_density
    rows_out = []
    cols_out = []
    for I in range(nbr):
        J = np.flatnonzero(keep[I])
        if J.size == 0:
            continue
        cols = (J[:, None] * b_col + np.arange(b_col)[None, :]).reshape(-1)
        cols = cols[cols < k]
        for r in range(I * b_row, min(m, (I + 1) * b_row)):
            c = cols
            if entry_density < 1.0:
                c = c[g.random(c.size) < entry_density]
            rows_out.append(np.full(c.size, r, np.int64))
            cols_out.append(c)
    rows = np.concatenate(rows_out) if rows_out else np.zeros(0, np.int64)
    cols = np.concatenate(cols_out) if cols_out else np.zeros(0, np.int64)
    cnt = np.bincount(rows, minlength=m) if m > 0 else np.zeros(0, np.int64)
    ptr = np.concatenate([[0], np.cumsum(cnt)])
    vals = _nonzero_values(rng_for(101, seed, 1, 0), cols.size, ab_dtype, _VALUE_DRAWS[kind])
    B = _b_draw(rng_for(101, seed, 2, 0), k, N, ab_dtype, kind)
    return _finish(f"blk_m{m}_k{k}_N{N}_s{seed}", m, k, N, ptr, cols, vals, B, ab_dtype, c_dtype,
                   "bcsr", b_row, b_col)

// gfx950 kernels for BCSR and WCSR SpMM (AsyncSparse paper, Sections III-A..III-C).
//
// Both formats reduce to the same per-tile computation.  A work-group tile owns
// R consecutive rows of C (a BCSR block row or a WCSR window, R = b_row) and a
// column slice of C.  Along the reduction the tile walks a "packed" column axis
// k':
//   BCSR  k' = q*b_col + kk  for the q-th stored block of the block row:
//         A(r, k') = blocks[q][r][kk],  B row = block_col_idx[q]*b_col + kk
//   WCSR  k' = p, a packed column of the window:
//         A(r, p)  = window tile[r][p],  B row = window_col_idx[p]  (-1 = pad)
// so the tile is a dense R x K' x BN product whose B operand is a row gather.
//
// MFMA mapping (v_mfma_f32_16x16x32_{f16,bf16}, wave64).  Lane l = 16*g + i
// supplies A[row i][k-group g] (8 consecutive k') and B[k-group g][column i];
// accumulator element q of lane l is D[4*g + q][i].  The k' rows of B are
// N-contiguous in memory while MFMA wants 8 consecutive k per lane, so every
// lane loads V consecutive columns of 8 gathered rows (one 2V-byte load per
// row) and transposes the 8 x V block in registers (v_perm_b32).  That gives
// the lane the B operand of V different 16x16 output tiles: in tile c, MFMA
// column i stands for C column  n_wave + i*V + c.  The accumulators of one lane
// therefore hold V adjacent columns of each of its rows, which the epilogue
// stores with one wide store per row.
//
// Memory access goes through buffer resources (base, size): a k' step past the
// end of the work item, a -1 pad column or an index outside [0, k) gets an
// offset beyond the resource size, and the hardware returns zeros.  There is no
// branch in the main loop and no access outside the caller's arrays.
//
// Latency hiding: every wave runs a two-stage software pipeline.  The B-row
// indices of step s+2 and the A/B data of step s+1 are in flight while the
// MFMAs of step s execute (vmcnt ordering keeps the later loads outstanding).
//
// Waves of a work-group split the tile's columns (waves_n, each 16*V wide) and
// the reduction (waves_k, interleaved 32-wide k' steps); the waves_k partial
// sums are added in a fixed order through LDS, so results are deterministic.
// WCSR tasks that cover only part of a long window write fp32 partial tiles to
// a workspace slot; wcsr_merge adds the slots of a window in a fixed order and
// rounds once (this replaces the paper's atomicAdd merge, Section III-C).
//
// Work-group order: dispatch hands consecutive work-group ids to the 8 XCDs in
// turn.  The kernel renumbers ids so that each XCD receives a contiguous range
// of (column tile, work item) pairs, column tile outermost: the work-groups
// that share a column slice of B run on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace wspmm {

// One pipeline stage: the gathered B rows and the A fragments of one k' step.
template <int MT, int DW>
struct Stage {
    uint32_t b[8][DW];
    u32x4_t a[MT];
};

// Steps of B/A loads kept in flight ahead of the MFMAs (1 to 3): as many as let
// the ring of D+1 register stages and the accumulators fit a register budget
// that leaves room for addressing at two waves per SIMD (256 VGPRs).  For
// 16-row tiles the budget stops at two steps: measured on the WCSR workloads,
// a third step in flight gains nothing.
template <int R, int V>
constexpr int pipe_depth()
{
    constexpr int acc = (R / 16) * V * 4;
    constexpr int stage = 8 * (V / 2) + (R / 16) * 4;
    constexpr int budget = R == 16 ? 140 : R == 32 ? 175 : 150;
    constexpr int ring = (budget - acc) / stage;  // stages that fit
    return ring >= 4 ? 3 : ring >= 2 ? ring - 1 : 1;
}

// Stores the V results of one row of one lane at byte offset `off` of r as DT
// (kOOB drops the store): V / 4 (fp32) or one (16-bit) store instructions,
// non-temporal (C is written once; measured: it then displaces less of the B
// rows that other work-groups still read from L2).
template <int V, int DT>
__device__ __forceinline__ void buf_store_row_dt(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *v)
{
    if constexpr (DT == SPMM_FP32) {
#pragma unroll
        for (int c = 0; c < V; c += 4)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4_t{__builtin_bit_cast(uint32_t, v[c]), __builtin_bit_cast(uint32_t, v[c + 1]),
                        __builtin_bit_cast(uint32_t, v[c + 2]), __builtin_bit_cast(uint32_t, v[c + 3])},
                r, (int)(off == kOOB ? kOOB : off + 4 * c), 0, kNT);
    } else if constexpr (V == 8) {
        u32x4_t w;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            w[c] = pack2(DT, v[2 * c], v[2 * c + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, kNT);
    } else {
        static_assert(V == 4, "16-bit rows of 4 or 8 values: one store");
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack2(DT, v[0], v[1]), pack2(DT, v[2], v[3])}, r,
                                              (int)off, 0, kNT);
    }
}

// Stores a 64-row accumulator tile of one lane as DT through rC (whose record 0
// is row row0 of C): rows 4g+q of each 16-row slice mt, V adjacent columns from
// ncol.  Rows past m and columns past N get out-of-range offsets.
template <int DT, int MT, int V>
__device__ __forceinline__ void store_acc_rows(const f32x4_t (&acc)[MT][V], __amdgpu_buffer_rsrc_t rC,
                                               int g, int64_t row0, int64_t m, int64_t ldc,
                                               int64_t ncol, int64_t N)
{
    constexpr int esz = DT == SPMM_FP32 ? 4 : 2;
    const bool col_ok = ncol < N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = mt * 16 + 4 * g + q;
            float v[V];
#pragma unroll
            for (int c = 0; c < V; ++c)
                v[c] = acc[mt][c][q];
            const bool ok = col_ok & (row0 + r < m);
            buf_store_row_dt<V, DT>(rC, ok ? (uint32_t)((r * ldc + ncol) * esz) : kOOB, v);
        }
}

// Column-major operands (B^T: N rows of k, C^T: N rows of m).  Lane (g, i) of
// MFMA column tile c holds column n = 16c + i of its tile; its results are rows
// 4g .. 4g+3 of each 16-row slice mt, four adjacent elements of C^T row n.
// Before the stores the four lanes (g = 0..3, same i) exchange their slices:
// a 4 x 4 transpose over (slice mt, lane group g), one v_permlane32_swap and one
// v_permlane16_swap stage per value, after which lane (g, i) holds rows
// 16g .. 16g+15 of column n, 16 adjacent elements of C^T row n, and writes them
// with 16-byte stores (two for 16-bit C, four for fp32) instead of one 8- or
// 16-byte store per slice.  Plain (not non-temporal) stores: the L2 joins the
// pieces of a line that the four lane groups write.  Measured on the gate_proj
// weight (column-major, bf16 C): 3368 us with one non-temporal store per slice,
// 2423 us with plain stores, 2163-2168 us exchanged and plain; down_proj 2381
// -> 2115 us.
// rC starts at a C^T row and ends `size` bytes later, after the last column
// (< N) the work-group may write, so columns past N fall outside it; tile_off
// (wave-uniform) is the byte offset of this tile's first C^T row inside rC.
// Rows past m are sent to offset size + ..., also outside (m is a multiple of
// 8, so a 16-byte store's four fp32 or eight 16-bit rows are all in or all
// out; the host keeps (N + 1024) * ldc * esz below 2^32, so no offset wraps).
// All 64 lanes must be active (the exchange reads other lanes).
template <int DT, int MT, int V>
__device__ __forceinline__ void store_acc_cm(const f32x4_t (&acc)[MT][V], __amdgpu_buffer_rsrc_t rC,
                                             uint32_t size, uint32_t tile_off, int g, int li,
                                             int64_t row0, int64_t m, int64_t ldc)
{
    static_assert(MT == 4, "four 16-row slices");
    constexpr int esz = DT == SPMM_FP32 ? 4 : 2;
    const uint32_t ldcb = (uint32_t)ldc * esz;
    const uint32_t lane_off = tile_off + (uint32_t)li * ldcb + (uint32_t)(row0 + 16 * g) * esz;
    const int32_t nrows = (int32_t)(m - row0 < (1 << 30) ? m - row0 : (1 << 30)) - 16 * g;
#pragma unroll
    for (int c = 0; c < V; ++c) {
        // x[h][q]: slice h of lane group g; after the exchange, row 16g + 4h + q
        // (each element is read into a scalar first: a bit cast of a vector
        // element expression compiles to a read of the vector's element 0)
        uint32_t x[4][4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float f = acc[h][c][q];
                x[h][q] = __builtin_bit_cast(uint32_t, f);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // lanes 32..63 of the first operand <-> lanes 0..31 of the second
            const auto a = __builtin_amdgcn_permlane32_swap(x[0][q], x[2][q], false, false);
            x[0][q] = a[0];
            x[2][q] = a[1];
            const auto b = __builtin_amdgcn_permlane32_swap(x[1][q], x[3][q], false, false);
            x[1][q] = b[0];
            x[3][q] = b[1];
            // lanes 16..31 and 48..63 of the first <-> 0..15 and 32..47 of the second
            const auto d = __builtin_amdgcn_permlane16_swap(x[0][q], x[1][q], false, false);
            x[0][q] = d[0];
            x[1][q] = d[1];
            const auto e = __builtin_amdgcn_permlane16_swap(x[2][q], x[3][q], false, false);
            x[2][q] = e[0];
            x[3][q] = e[1];
        }
        const uint32_t base = lane_off + (uint32_t)(16 * c) * ldcb;
        if constexpr (DT == SPMM_FP32) {
#pragma unroll
            for (int h = 0; h < 4; ++h)
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{x[h][0], x[h][1], x[h][2], x[h][3]}, rC,
                                                       (int)(4 * h < nrows ? base + 16u * h : size), 0, 0);
        } else {
            const auto pk = [&](uint32_t lo, uint32_t hi) {
                return pack2(DT, __builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
            };
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4_t{pk(x[2 * j][0], x[2 * j][1]), pk(x[2 * j][2], x[2 * j][3]),
                            pk(x[2 * j + 1][0], x[2 * j + 1][1]), pk(x[2 * j + 1][2], x[2 * j + 1][3])},
                    rC, (int)(8 * j < nrows ? base + 16u * j : size), 0, 0);
        }
    }
}

template <int MT, int V>
__device__ __forceinline__ void store_tile_cm(int dt, const f32x4_t (&acc)[MT][V],
                                              __amdgpu_buffer_rsrc_t rC, uint32_t size,
                                              uint32_t tile_off, int g, int li, int64_t row0,
                                              int64_t m, int64_t ldc)
{
    if (dt == SPMM_FP32)
        store_acc_cm<SPMM_FP32>(acc, rC, size, tile_off, g, li, row0, m, ldc);
    else if (dt == SPMM_BF16)
        store_acc_cm<SPMM_BF16>(acc, rC, size, tile_off, g, li, row0, m, ldc);
    else
        store_acc_cm<SPMM_FP16>(acc, rC, size, tile_off, g, li, row0, m, ldc);
}

// Stores the V results of one row of one lane (V adjacent columns) at byte
// offset `off` of r; kOOB drops the store.  For a given V both the fp32 and the
// 16-bit forms issue the same number of store instructions, so wait counts on
// loads issued before the stores stay exact whatever the destination.  The
// stores are non-temporal: C (and a partial tile) is written once, and kept out
// of the way it displaces less of the B rows other work-groups still gather
// (measured: 42.6-44.0 -> 41.3-41.5 us on the 65536^2 BCSR P*V workload, 4 %
// on small WCSR matrices, no change on the 16384^2 WCSR one).
template <int V>
__device__ __forceinline__ void buf_store_row(__amdgpu_buffer_rsrc_t r, uint32_t off, int dt,
                                              const float *v)
{
    if (dt == SPMM_FP32) {
        if constexpr (V >= 4) {
#pragma unroll
            for (int c = 0; c < V; c += 4)
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4_t{__builtin_bit_cast(uint32_t, v[c]), __builtin_bit_cast(uint32_t, v[c + 1]),
                            __builtin_bit_cast(uint32_t, v[c + 2]), __builtin_bit_cast(uint32_t, v[c + 3])},
                    r, (int)(off == kOOB ? kOOB : off + 4 * c), 0, kNT);
        } else {
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2_t{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1])}, r,
                (int)off, 0, kNT);
        }
    } else {
        uint32_t w[V / 2];
#pragma unroll
        for (int c = 0; c < V; c += 2)
            w[c / 2] = pack2(dt, v[c], v[c + 1]);
        if constexpr (V == 8) {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{w[0], w[1], w[2], w[3]}, r, (int)off, 0, kNT);
            __builtin_amdgcn_raw_buffer_store_b32(0u, r, (int)kOOB, 0, kNT);  // count filler
        } else if constexpr (V == 4) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w[0], w[1]}, r, (int)off, 0, kNT);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(w[0], r, (int)off, 0, kNT);
        }
    }
}

// Wave-uniform state of one task of the tile kernel (raw fields; buffer
// resources are rebuilt where they are used).
struct TaskCtx {
    const uint16_t *a;   // A values of the task's row tile (BCSR: its first block;
                         // WCSR: its window in the plan's fragment-order copy)
    uint32_t klen;       // packed columns (0: nothing to load)
    uint32_t begin;      // first packed column (counted from the start of the format)
    uint32_t width;      // WCSR window width (A row pitch); BCSR: b_col
    uint32_t a_col0;     // WCSR: the task's first packed column inside its window
    int32_t tile;        // row tile
    int32_t slot;        // partial slot, or -1: the task writes C
    int32_t ctile;       // column tile
    uint32_t lds;        // first int of the task's LDS index buffer
};

// Generic tile kernel.  A task is a row tile (a BCSR block row or a WCSR window)
// and a range of its packed columns; a work item is a (task, column tile) pair.
// The grid is persistent: work-group b runs the items of its own list, entries
// list[b] .. list[b+1]-1 of the descriptor table, which the host fills by
// greedy longest-first assignment of the items to the least loaded work-group.
//   * Two LDS index buffers.  While a task runs, its waves copy the B-row
//     indices (WCSR column indices or BCSR block columns) of the next task into
//     the other buffer with direct-to-LDS loads, one copy per ring iteration;
//     the next descriptor (8 ints, lane j holds int j) is loaded a task ahead.
//   * Each wave keeps D steps of A/B loads in flight in a ring of D+1 register
//     stages.  The ring runs across tasks: the last iteration of a task issues
//     the first D steps of the next one, so the pipeline fills once per
//     work-group.
//   * Every task issues the same branch-free sequence of vector memory
//     instructions (loads past a task's end and stores that are masked off use
//     out-of-range offsets), so the compiler's wait counts stay exact and loads
//     of the next task are never waited for behind the stores of this one.
//   * Tasks that cover part of a row tile write an fp32 partial slot; the
//     waves_k partial sums are added in a fixed order through LDS.
template <int FMT, int R, int V, int AB>
__global__ __launch_bounds__(256, 2) void spmm_tile_kernel(TileParams p)
{
    constexpr int MT = R / 16;           // 16-row MFMA tiles per work-group tile
    constexpr int DW = V / 2;            // dwords of one gathered row segment per lane
    constexpr int D = pipe_depth<R, V>();
    constexpr int Q = D + 1;
    constexpr int kStageOps = 8 + MT;    // vector memory instructions per ring stage
    constexpr uint32_t RUN = FMT == 1 ? 256 : 64;  // index ints per direct-to-LDS copy
    // Wave priority while a wave issues its loads (0: unchanged).  64-row tiles
    // (one step in flight per wave) raise it so that a wave ready to issue is
    // not held behind other waves' MFMAs (measured: 65536^2 BCSR P*V 34.3-35.8
    // -> 33.4-33.7 us; no gain on 16-row WCSR tiles).
    constexpr int kIssuePrio = R == 64 ? 1 : 0;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int32_t *const lds = reinterpret_cast<int32_t *>(smem);
    typedef __attribute__((address_space(3))) void lds_void;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % p.waves_n;
    const int wk = wave / p.waves_n;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int nwaves = p.waves_n * p.waves_k;

    // This work-group's entries of the descriptor table: lists[b] .. lists[b+1]-1.
    const uint32_t first = (uint32_t)p.lists[blockIdx.x];
    const uint32_t limit = (uint32_t)p.lists[blockIdx.x + 1];
    // LDS: index buffer 0 (buf_ints ints), a 256-int sink for copies that
    // carry nothing, the cross-wave reduction area (waves_k > 1), then index
    // buffer 1, which the host leaves out when every work-group runs one entry
    constexpr int NR = 4 * MT * V;  // accumulator floats per lane
    const uint32_t buf_ints = (uint32_t)p.lds_idx_ints;
    const uint32_t sink = buf_ints;
    const uint32_t red_ints = p.waves_k > 1 ? (uint32_t)(nwaves * NR * 64) : 0u;
    const uint32_t buf1 = buf_ints + 256 + red_ints;
    const uint32_t idx_cap = buf_ints - 8;               // last valid start of an index read

    // Descriptor of entry e: lane l < 8 holds int l (zeros for an invalid entry).
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(p.tasks, (uint32_t)(p.n_entries * 32));
    auto load_desc = [&](uint32_t e) -> uint32_t {
        return __builtin_amdgcn_raw_buffer_load_b32(
            rT, e < limit ? (e * 8u + (uint32_t)(lane & 7)) * 4u : kOOB, 0, 0);
    };
    auto make_ctx = [&](uint32_t dv, uint32_t buf) {
        TaskCtx c;
        c.tile = __builtin_amdgcn_readlane((int)dv, 0);
        c.begin = (uint32_t)__builtin_amdgcn_readlane((int)dv, 1);
        c.klen = (uint32_t)__builtin_amdgcn_readlane((int)dv, 2) - c.begin;
        c.slot = __builtin_amdgcn_readlane((int)dv, 3);
        c.ctile = __builtin_amdgcn_readlane((int)dv, 6);
        c.lds = buf ? buf1 : 0u;
        if constexpr (FMT == 0) {
            c.a = p.A + ((int64_t)c.begin >> p.log2_b_col) * R * p.b_col;
            c.width = (uint32_t)p.b_col;
            c.a_col0 = 0;
        } else {
            const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)dv, 4);
            c.a = p.A + (int64_t)R * (uint32_t)__builtin_amdgcn_readlane((int)dv, 7);
            c.width = (uint32_t)__builtin_amdgcn_readlane((int)dv, 5);
            c.a_col0 = c.begin - base;
        }
        return c;
    };
    // The empty task: loads nothing (every offset out of range), stores nothing.
    auto null_ctx = [&](const TaskCtx &like) {
        TaskCtx c = like;
        c.klen = 0;
        return c;
    };
    auto n_idx_of = [&](const TaskCtx &c) -> uint32_t {
        if constexpr (FMT == 0)
            return c.klen >> p.log2_b_col;
        else
            return c.klen;
    };
    auto nit_of = [&](const TaskCtx &c) -> int32_t {
        const uint32_t steps0 = (c.klen + 32u * p.waves_k - 1) / (32u * p.waves_k);  // wave 0's
        return (int32_t)((steps0 + Q - 1) / Q);
    };
    auto col0_of = [&](const TaskCtx &c) -> int64_t {
        return (int64_t)c.ctile * p.tile_cols + wn * 16 * V;
    };
    // Copy r of a task's indices into its buffer (a dummy copy into the sink if
    // the task has no run r or `enable` is false).
    auto copy_run = [&](const TaskCtx &c, uint32_t r, bool enable = true) {
        const uint32_t n_idx = n_idx_of(c);
        const int32_t *gidx = p.col_idx + (FMT == 0 ? (c.begin >> p.log2_b_col) : c.begin);
        const __amdgpu_buffer_rsrc_t rI = make_rsrc(gidx, n_idx * 4u);
        const bool real = enable & (r < (n_idx + RUN - 1) / RUN);
        const uint32_t dst = real ? c.lds + r * RUN : sink;
        if constexpr (FMT == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rI, (lds_void *)(lds + dst), 16,
                                                     real ? (r * 64u + lane) * 16u : kOOB, 0, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rI, (lds_void *)(lds + dst), 4,
                                                     real ? (r * 64u + lane) * 4u : kOOB, 0, 0, 0);
    };
    auto n_runs = [&](const TaskCtx &c) { return (n_idx_of(c) + RUN - 1) / RUN; };

    const uint32_t ldb2 = (uint32_t)p.ldb * 2;
    const uint32_t lane_col_bytes = (uint32_t)li * V * 2;
    const uint32_t k32 = (uint32_t)p.k;
    const uint32_t nbc = (uint32_t)((p.k + p.b_col - 1) >> p.log2_b_col);  // block columns
    // this lane's first packed column (task-relative) at step s: kfirst + s * kstride
    const uint32_t kfirst = 32u * wk + 8u * g;
    const uint32_t kstride = 32u * p.waves_k;

    f32x4_t acc[MT][V];

    // Issues the A and B loads of step s of task c into st.
    auto issue = [&](const TaskCtx &c, int s, Stage<MT, DW> &st) {
        const uint32_t kl = kfirst + (uint32_t)s * kstride;  // task-relative packed column
        const bool ok = kl < c.klen;
        const int32_t *lidx = lds + c.lds;
        const int64_t col0 = col0_of(c);
        const uint64_t b_skip = (uint64_t)col0 * 2;
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(p.B + col0, (uint32_t)(p.b_bytes > b_skip ? p.b_bytes - b_skip : 0));
        // BCSR: row-major b_row x b_col blocks.  WCSR: the plan's copy, one
        // 1 KB fragment per (32-column step, 16 rows): lane l reads bytes
        // 16l .. 16l+15 of fragment mt of step (a_col0 + kl) / 32 (tasks start
        // on step boundaries), so every A load is one contiguous 1 KB run
        // (measured on the 16384^2 WCSR workload against 16 half lines per load
        // in the row-major window tile: 39.1-39.3 against 41.8-42.0 us warm)
        const uint32_t a_row_stride = FMT == 0 ? (uint32_t)p.b_col * 2u : 0u;
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(c.a, FMT == 0 ? n_idx_of(c) * (uint32_t)(R * p.b_col * 2)
                                    : (uint32_t)R * ((c.width + 31u) & ~31u) * 2u);
        // A fragments first, then the B rows: the MFMAs of a stage wait for its
        // last B row, which also covers its A
        const uint32_t q = kl >> p.log2_b_col;            // BCSR: block of the task
        const uint32_t kk = kl & (uint32_t)(p.b_col - 1);  // BCSR: column in the block
        const uint32_t a_off = FMT == 0 ? ((q * R + li) * (uint32_t)p.b_col + kk) * 2u
                                        : ((c.a_col0 + kl) >> 5) * (uint32_t)(R * 64) + (uint32_t)lane * 16u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            uint32_t w[4];
            const uint32_t mt_off = FMT == 0 ? (uint32_t)(mt * 16) * a_row_stride : (uint32_t)mt * 1024u;
            buf_load<4>(rA, ok ? a_off + mt_off : kOOB, w);
            st.a[mt] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
        if constexpr (FMT == 0) {
            const uint32_t J = (uint32_t)lidx[q < idx_cap ? q : idx_cap];  // in-bounds read
            const bool jv = ok & (J < nbc);
            const uint32_t r0 = (jv ? J : 0u) * (uint32_t)p.b_col + kk;
            // rows r0 .. r0+7 are consecutive: one 24-bit multiply, then + j*ldb2
            const uint32_t base = __umul24(r0, ldb2) + lane_col_bytes;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                buf_load<DW>(rB, (jv & (r0 + j < k32)) ? base + (uint32_t)j * ldb2 : kOOB, st.b[j]);
        } else {
            const uint32_t kr = kl < idx_cap ? kl : idx_cap;  // in-bounds LDS read
            const u32x4_t i0 = *reinterpret_cast<const u32x4_t *>(lidx + kr);
            const u32x4_t i1 = *reinterpret_cast<const u32x4_t *>(lidx + kr + 4);
            const uint32_t ix[8] = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t r = ix[j];
                // (k < 2^24 and ldb * 2 < 2^24: the host checks both)
                buf_load<DW>(rB, (ok & (r < k32)) ? __umul24(r, ldb2) + lane_col_bytes : kOOB, st.b[j]);
            }
        }
    };

    auto compute = [&](const Stage<MT, DW> &st) {
#pragma unroll
        for (int c = 0; c < V; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t bf;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bf[q] = __builtin_amdgcn_perm(st.b[2 * q + 1][c >> 1], st.b[2 * q][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(st.a[mt], bf, acc[mt][c]);
        }
    };

    // Finishes task c: with waves_k > 1 every wave writes its partial tile to
    // its own slice of the reduction area, and after one barrier each wave adds
    // the waves_k partials of a quarter (waves_k = 4), a half (2) or all of the
    // tile rows, in wave order (the same sum whichever wave does it), and stores
    // those rows: rows 4g+q of each 16-row tile, V adjacent columns per lane.
    // Every wave issues the same stores; rows it does not own, rows past m and
    // columns past N get out-of-range offsets.
    float *const red = reinterpret_cast<float *>(lds + buf_ints + 256);
    auto finish = [&](const TaskCtx &c, bool real) {
        const int qn = 4 / p.waves_k;   // rows q this wave stores: [q0, q0 + qn)
        const int q0 = wk * qn;
        if (real && p.waves_k > 1) {
            float *mine = red + wave * NR * 64 + lane;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int cc = 0; cc < V; ++cc)
                        mine[((q * MT + mt) * V + cc) * 64] = acc[mt][cc][q];
            lds_barrier();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q < q0 || q >= q0 + qn)
                    continue;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int cc = 0; cc < V; ++cc) {
                        const int e = ((q * MT + mt) * V + cc) * 64 + lane;
                        // waves_k is 2 or 4 here: partials of waves wn, wn + waves_n, ...
                        float sum = red[wn * NR * 64 + e];
                        sum += red[(p.waves_n + wn) * NR * 64 + e];
                        if (p.waves_k > 2) {
                            sum += red[(2 * p.waves_n + wn) * NR * 64 + e];
                            sum += red[(3 * p.waves_n + wn) * NR * 64 + e];
                        }
                        acc[mt][cc][q] = sum;
                    }
            }
        }
        const bool to_partial = c.slot >= 0;
        const int64_t row0 = (int64_t)c.tile * R;
        const int64_t col0 = col0_of(c);
        const int dt = to_partial ? SPMM_FP32 : p.c_dtype;
        const uint32_t esz = dt == SPMM_FP32 ? 4u : 2u;
        const int64_t stride = to_partial ? p.N : p.ldc;  // elements between rows
        void *base = to_partial ? (void *)(p.partial + ((int64_t)c.slot * R * p.N + col0))
                                : (void *)((uint8_t *)p.C + (row0 * p.ldc + col0) * esz);
        const __amdgpu_buffer_rsrc_t rO = make_rsrc(base, (uint32_t)(R * stride) * esz);
        const bool lane_ok = real & (col0 + li * V < p.N);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = mt * 16 + 4 * g + q;
                float v[V];
#pragma unroll
                for (int cc = 0; cc < V; ++cc)
                    v[cc] = acc[mt][cc][q];
                const bool mine_q = (q >= q0) & (q < q0 + qn);
                const bool row_ok = to_partial | (row0 + r < p.m);
                const uint32_t off = (lane_ok & mine_q & row_ok)
                                         ? ((uint32_t)r * (uint32_t)stride + li * V) * esz
                                         : kOOB;
                buf_store_row<V>(rO, off, dt, v);
            }
        }
    };

    // ---- entries of the first three turns -----------------------------------
    const uint32_t e0 = first;
    uint32_t e_next = first + 1, e_next2 = first + 2;
    if (e0 >= limit)
        return;

    // ---- first task: indices staged before the ring starts ----------------
    TaskCtx cur = make_ctx(load_desc(e0), 0);
    for (uint32_t r = wave; r < n_runs(cur); r += nwaves)
        copy_run(cur, r);
    uint32_t d_next = load_desc(e_next);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    Stage<MT, DW> st[Q];
#pragma unroll
    for (int u = 0; u < D; ++u)
        issue(cur, u, st[u]);

    TaskCtx prev = cur;
    bool have_prev = false;
    for (uint32_t j = 0;; ++j) {
        // ---- finish the previous task (its last steps ran in the last turn) ----
        finish(prev, have_prev);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int c = 0; c < V; ++c)
                acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const bool has_next = e_next < limit;
        const TaskCtx nxt = has_next ? make_ctx(d_next, (j + 1) & 1) : null_ctx(cur);
        const uint32_t d_next2 = load_desc(e_next2);

        // ---- the task's steps.  Every iteration issues one index copy of the
        // next task and Q ring stages; in the last one the copy is a dummy and
        // the stages beyond this task's end are the next task's first D. ----
        const int32_t nit_cur = nit_of(cur);
        const uint32_t copied = nit_cur > 1 ? (uint32_t)(nit_cur - 1) * nwaves : 0u;
        // The next task's indices must be in LDS before its first issue; the
        // barrier also ends every wave's reads of this task's buffer, which the
        // copies for the task after next overwrite.
        auto boundary = [&]() {
            if (n_runs(nxt) > copied) {
                for (uint32_t r = copied + wave; r < n_runs(nxt); r += nwaves)
                    copy_run(nxt, r);
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            } else {
                // every real copy was followed by more than D ring stages
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(D * kStageOps));
            }
            lds_barrier();
        };
        int s = 0;
        for (int it = 0; it < nit_cur; ++it, s += Q) {
            const bool last = it + 1 == nit_cur;
            copy_run(nxt, (uint32_t)(it * nwaves + wave), !last);
#pragma unroll
            for (int u = 0; u < Q; ++u) {
                if (u == Q - D) {
                    // this task's indices have been read for the last time;
                    // from here on the last iteration reads the next task's
                    __builtin_amdgcn_sched_barrier(0);
                    if (last)
                        boundary();
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kIssuePrio > 0)
                    __builtin_amdgcn_s_setprio(kIssuePrio);
                if (u + D < Q) {
                    issue(cur, s + u + D, st[(u + D) % Q]);
                } else {
                    // wave-uniform selection between this task's step and the next's
                    TaskCtx c = last ? nxt : cur;
                    issue(c, last ? u + D - Q : s + u + D, st[(u + D) % Q]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kIssuePrio > 0)
                    __builtin_amdgcn_s_setprio(0);
                compute(st[u]);  // steps past the end hold zeros
            }
        }
        if (nit_cur == 0) {
            boundary();
#pragma unroll
            for (int u = 0; u < D; ++u)
                issue(nxt, u, st[u]);
        }
        prev = cur;
        have_prev = true;
        if (!has_next)
            break;
        cur = nxt;
        d_next = d_next2;
        e_next = e_next2;
        e_next2 = e_next2 + 1;
    }
    finish(prev, true);
}

// BCSR with 64 x 64 blocks and a wide column tile (NW waves x 16V columns).
// Same MFMA mapping and B pipeline as spmm_tile_kernel, but the A block is
// shared: the work-group loads each 64 x 64 block once into one of two LDS
// buffers (MFMA fragment order), and every wave reads its A fragments from
// there.  Block-column indices are work-group uniform and come through scalar
// loads.  One LDS barrier per block.  CM: column-major B and C (B^T and C^T
// row-major), 4 columns per lane: a whole block of B^T lines per stage,
// regrouped through a per-wave LDS scratch as in bcsr64_sweep_kernel.
template <int AB, int NW, bool CM>
__global__ __launch_bounds__(NW * 64) void bcsr64_lds_kernel(TileParams p,
                                                             const int32_t *__restrict__ block_cols)
{
    constexpr int R = 64, BC = 64, MT = 4, V = CM ? 4 : 8, DW = 4;
    constexpr int NT = NW * 64;                    // threads per work-group
    // A buffers in MFMA fragment order: the 16 bytes lane l = 16g + i reads for
    // (k half h, row slice mt) -- row 16mt + i, k = 32h + 8g .. +7 -- sit at
    // ((h * 4 + mt) * 64 + l) * 16, so that every LDS write and every fragment
    // read is one contiguous 1 KB run (no bank conflicts; padded rows read as
    // 16 rows x 16 bytes took 3.2 conflict cycles per LDS instruction)
    constexpr int ABUF = R * BC * 2;               // bytes of one A buffer
    constexpr int CPT = R * BC / 8 / NT;           // 16-byte chunks per thread per block
    constexpr bool A_FRAG = NW == 1 && !CM;        // A from the plan's fragment-order copy
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * ABUF];
    __shared__ __attribute__((aligned(16))) uint8_t lds_scr[CM ? NW * kSweepCmScratch : 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;

    int64_t item, ctile;
    tile_of(p.n_items, p.n_items * p.n_col_tiles, p.order, item, ctile);
    const int64_t blk0 = p.row_ptr[item];
    const int nblk = p.row_ptr[item + 1] - (int)blk0;
    const int64_t row0 = item * R;
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A + blk0 * R * BC, (uint32_t)((int64_t)nblk * R * BC * 2));
    const int64_t col0 = ctile * p.tile_cols + wave * 16 * V;
    // row-major: B + col0 (column col0 of every row); CM: B^T row col0
    const uint64_t b_skip = CM ? (uint64_t)col0 * p.ldb * 2 : (uint64_t)col0 * 2;
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(
        p.B + (CM ? col0 * p.ldb : col0), (uint32_t)(p.b_bytes > b_skip ? p.b_bytes - b_skip : 0));
    const uint32_t ldb2 = (uint32_t)p.ldb * 2;
    const uint32_t lane_col_bytes = (uint32_t)li * V * 2;
    const uint32_t k32 = (uint32_t)p.k;
    const uint32_t nbc = (uint32_t)((p.k + BC - 1) / BC);

    f32x4_t acc[MT][V];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < V; ++c)
            acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // cooperative A-block copy in fragment order: chunk c = (h * MT + mt) * 64 + l,
    // lane l = 16g + i: row 16mt + i, k = 32h + 8g .. +7.  The one-wave
    // row-major form reads the plan's copy, already in that order (each load
    // one contiguous 1 KB run; measured on the 65536^2 P*V workload: 29.5-29.8
    // against 30.3-30.6 us warm); the others read the caller's row-major blocks
    // (16 rows of 64 bytes per load; on down_proj the copy gained nothing).
    auto load_a = [&](int q, u32x4_t (&r)[CPT]) {
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const int c = threadIdx.x + t * NT;
            const int l = c & 63, hm = c >> 6;
            const int row = 16 * (hm % MT) + (l & 15), cc = 4 * (hm / MT) + (l >> 4);
            // plain loads: A is read again for every column tile and is small
            // enough to stay in the memory-side cache; non-temporal loads, which
            // do not keep it there, made down_proj 8 % slower (1605 against
            // 1472-1481 us)
            const uint32_t off = A_FRAG ? (uint32_t)q * R * BC * 2 + (uint32_t)c * 16
                                        : ((uint32_t)q * R * BC + (uint32_t)row * BC + (uint32_t)cc * 8) * 2;
            r[t] = __builtin_amdgcn_raw_buffer_load_b128(rA, (int)off, 0, 0);
        }
    };
    auto store_a = [&](int buf, const u32x4_t (&r)[CPT]) {
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const int c = threadIdx.x + t * NT;
            *reinterpret_cast<u32x4_t *>(lds_a + buf * ABUF + c * 16) = r[t];
        }
    };
    // Block column of block q (work-group uniform, so a scalar load); -1 past the end.
    auto block_col = [&](int q) -> uint32_t {
        const int at = __builtin_amdgcn_readfirstlane((int)blk0 + (q < nblk ? q : 0));
        const uint32_t J = (uint32_t)block_cols[at];
        return q < nblk ? J : 0xFFFFFFFFu;
    };
    // Row-major: k' step s of block column J (half s%2), B rows J*64 + 32*(s%2) +
    // 8g + j.  CM: the whole block (k is a multiple of 8: a lane's eight values
    // are all inside B^T's row or all past it).
    auto issue_b = [&](int s, uint32_t J, BStage<DW> &st) {
        const bool jv = J < nbc;
        if constexpr (CM) {
            // the whole block of the wave's 64 B^T rows as 8 whole 128-byte
            // lines per load: load e brings rows 8e .. 8e+7 (row 8e + lane/8,
            // the 16 bytes of k = J*64 + 8*(lane%8) .. +7); `s` is unused
            const uint32_t kq = (jv ? J : 0u) * BC + 8 * (uint32_t)(lane & 7);
            const uint32_t base = (uint32_t)(lane >> 3) * ldb2 + kq * 2;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                buf_load<DW>(rB, (jv & (kq < k32)) ? base + (uint32_t)(8 * e) * ldb2 : kOOB, st.b[e]);
        } else {
            const uint32_t r0 = (jv ? J : 0u) * BC + (uint32_t)(s & 1) * 32 + 8 * g;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t r = r0 + j;
                buf_load<DW>(rB, (jv & (r < k32)) ? r * ldb2 + lane_col_bytes : kOOB, st.b[j]);
            }
        }
    };
    // row-major half-block (column-major blocks go through compute_cm)
    auto compute = [&](const BStage<DW> &st, int buf, int half) {
        u32x4_t af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            af[mt] = *reinterpret_cast<const u32x4_t *>(lds_a + buf * ABUF +
                                                       ((half * MT + mt) * 64 + lane) * 16);
#pragma unroll
        for (int c = 0; c < V; ++c) {
            u32x4_t bf;
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bf[q] = __builtin_amdgcn_perm(st.b[2 * q + 1][c >> 1], st.b[2 * q][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(af[mt], bf, acc[mt][c]);
        }
    };
    // CM, one whole block from buffer `buf`: the lines of column group c (16
    // rows) pass through the wave's scratch, chunk x of row r at slot
    // x ^ (r % 8), and lane (g, i) of half h reads chunk 4h + g of row i (no
    // bank conflicts within an 8-lane read phase; the scratch is the wave's
    // own and its LDS instructions complete in order)
    uint8_t *const scr = lds_scr + (CM ? wave * kSweepCmScratch : 0);
    auto compute_cm = [&](const BStage<DW> &st, int buf) {
        u32x4_t af[2][MT];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[hh][mt] = *reinterpret_cast<const u32x4_t *>(lds_a + buf * ABUF +
                                                               ((hh * MT + mt) * 64 + lane) * 16);
#pragma unroll
        for (int c = 0; c < V; ++c) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                *reinterpret_cast<u32x4_t *>(scr + (8 * e + (lane >> 3)) * 128 +
                                             (((lane & 7) ^ (lane >> 3)) * 16)) =
                    u32x4_t{st.b[2 * c + e][0], st.b[2 * c + e][1], st.b[2 * c + e][2],
                            st.b[2 * c + e][3]};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4_t bf = *reinterpret_cast<const u32x4_t *>(
                    scr + li * 128 + (((4 * hh + g) ^ (li & 7)) * 16));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][c] = mfma16x16x32<AB>(af[hh][mt], bf, acc[mt][c]);
            }
        }
    };

    if (CM && nblk > 0) {
        // two blocks per iteration: st0 and A buffer 0 hold block q, st1 and
        // buffer 1 block q + 1 (past the row's end: zeros, not computed); every
        // path issues the same loads, which keeps the wait counts exact
        u32x4_t areg[CPT];
        BStage<DW> st0, st1;
        load_a(0, areg);
        issue_b(0, block_col(0), st0);
        store_a(0, areg);
        lds_barrier();
        for (int q = 0; q < nblk; q += 2) {
            issue_b(0, block_col(q + 1), st1);
            load_a(q + 1 < nblk ? q + 1 : q, areg);
            __builtin_amdgcn_sched_barrier(0);
            compute_cm(st0, 0);
            __builtin_amdgcn_sched_barrier(0);
            store_a(1, areg);
            lds_barrier();
            issue_b(0, block_col(q + 2), st0);
            load_a(q + 2 < nblk ? q + 2 : q, areg);
            __builtin_amdgcn_sched_barrier(0);
            if (q + 1 < nblk)
                compute_cm(st1, 1);
            __builtin_amdgcn_sched_barrier(0);
            store_a(0, areg);
            lds_barrier();
        }
    } else if (nblk > 0) {
        u32x4_t areg[CPT];
        BStage<DW> st0, st1;
        uint32_t Jcur = block_col(0);
        load_a(0, areg);
        issue_b(0, Jcur, st0);
        store_a(0, areg);
        lds_barrier();
        for (int q = 0; q < nblk; ++q) {
            // first half of block q: prefetch its second half, the next A block and
            // the next block column
            const uint32_t Jnext = block_col(q + 1);
            issue_b(1, Jcur, st1);
            load_a(q + 1 < nblk ? q + 1 : q, areg);
            __builtin_amdgcn_sched_barrier(0);
            compute(st0, q & 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            // second half: prefetch the first half of block q+1
            issue_b(0, Jnext, st0);
            __builtin_amdgcn_sched_barrier(0);
            compute(st1, q & 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            store_a((q + 1) & 1, areg);
            lds_barrier();
            Jcur = Jnext;
        }
    }

    // epilogue: one branch on C's type, non-temporal stores
    const int esz = p.c_dtype == SPMM_FP32 ? 4 : 2;
    if constexpr (CM) {
        const int64_t n_end = col0 + 16 * V < p.N ? col0 + 16 * V : p.N;
        const uint32_t size = n_end > col0 ? (uint32_t)((n_end - col0) * p.ldc * esz) : 0u;
        const __amdgpu_buffer_rsrc_t rCt = make_rsrc((uint8_t *)p.C + col0 * p.ldc * esz, size);
        store_tile_cm(p.c_dtype, acc, rCt, size, 0u, g, li, row0, p.m, p.ldc);
        return;
    }
    const int64_t ncol = col0 + li * V;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc((uint8_t *)p.C + row0 * p.ldc * esz, (uint32_t)(R * p.ldc * esz));
    if (p.c_dtype == SPMM_FP32)
        store_acc_rows<SPMM_FP32>(acc, rC, g, row0, p.m, p.ldc, ncol, p.N);
    else if (p.c_dtype == SPMM_BF16)
        store_acc_rows<SPMM_BF16>(acc, rC, g, row0, p.m, p.ldc, ncol, p.N);
    else
        store_acc_rows<SPMM_FP16>(acc, rC, g, row0, p.m, p.ldc, ncol, p.N);
}

// BCSR with 64 x 64 blocks, wide N and at most kSweepMaxBlocks blocks per
// block row: the A blocks stay put and the B tiles move.  A work-group loads
// every block of its block row into padded LDS rows once, then sweeps a
// contiguous range of column tiles (NW waves x 128 columns each) with no
// further barrier: per tile it zeroes its accumulators, walks the blocks with
// the same two-stage B pipeline as bcsr64_lds_kernel (the pipeline runs on
// across tile boundaries) and stores the tile.  Launch order deals work-groups
// to the XCDs in turn; XCD x runs the column ranges x, x + 8, ... and, inside a
// range, the block rows in order, so the work-groups resident on one XCD sweep
// the same column tiles at about the same time and share each tile's B rows in
// that XCD's L2, and A is read once per (block row, range).  CM: column-major B
// and C, as in bcsr64_lds_kernel.  VR: row-major columns per lane (8, or 4 for
// 256-column tiles, whose B column slices take half the L2).
template <int AB, int NW, bool CM, int VR>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 1 : 2) void bcsr64_sweep_kernel(TileParams p)
{
    // CM: 4 columns per lane, so that a whole block of B^T (both halves) fits
    // one ring stage.  F8: one-byte codes (8 columns per lane = 2 dwords per row)
    constexpr bool F8 = AB == SPMM_FP8_E4M3;
    static_assert(!(F8 && CM) && !(F8 && VR != 8), "fp8 runs with row-major B and C, 8 columns per lane");
    static_assert(VR == 8 || (VR == 4 && !CM), "4 or 8 row-major columns per lane");
    constexpr int ESZ = F8 ? 1 : 2;                // bytes per A / B element
    constexpr int R = 64, BC = 64, MT = 4, V = CM ? 4 : VR;
    constexpr int DW = CM ? 4 : V * ESZ / 4;       // dwords of one B row segment per lane
    constexpr int NT = NW * 64;
    // Padded LDS rows, filled with row-major loads.  The fragment reads take
    // about 3.6 bank-conflict cycles per LDS instruction; the conflict-free
    // fragment order of bcsr64_lds_kernel, whose A loads are then strided, made
    // this kernel 5 % slower (its A is loaded at every work-group's start, on
    // the critical path; the LDS itself is not)
    constexpr int STRIDE = BC * ESZ + 16;
    constexpr int ABUF = R * STRIDE;               // bytes of one block in LDS
    constexpr int CPR = BC * ESZ / 16;             // 16-byte chunks per block row
    constexpr int CPB = R * CPR;                   // 16-byte chunks per block
    constexpr int MAXC = kSweepMaxBlocks * CPB / NT;  // chunks per thread, fullest row
    // CM: a per-wave scratch of 16 B^T rows x 128 bytes in front of the A blocks
    constexpr int SCR = CM ? kSweepCmScratch : 0;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    uint8_t *const lds_a = lds_dyn + NW * SCR;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;
    uint8_t *const scr = lds_dyn + wave * SCR;

    const uint32_t xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const uint32_t h = local / (uint32_t)p.n_items;
    const uint32_t item = __builtin_amdgcn_readfirstlane(local - h * (uint32_t)p.n_items);
    const int64_t t_begin = (int64_t)(h * 8 + xcd) * p.range_tiles;
    const int64_t t_end = t_begin + p.range_tiles < p.n_col_tiles ? t_begin + p.range_tiles
                                                                  : p.n_col_tiles;
    if (t_begin >= t_end)
        return;  // the whole work-group
    const int ntiles = (int)(t_end - t_begin);
    const int64_t blk0 = p.row_ptr[item];
    const int nblk = p.row_ptr[item + 1] - (int)blk0;  // <= kSweepMaxBlocks (the plan checks)
    const int64_t row0 = (int64_t)item * R;

    // the block row's A blocks -> LDS: every load in flight before the first store.
    // Plain loads: every column range reads A again, and A (a few to a few tens
    // of MB) stays in the memory-side cache between them; with non-temporal
    // loads gate_proj ran 7 % slower (1408-1425 against 1309-1319 us). A costs
    // about 400 us of the launch either way (1015-1020 us with its loads
    // skipped, timing only).
    {
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(
            reinterpret_cast<const uint8_t *>(p.A) + blk0 * R * BC * ESZ, (uint32_t)(nblk * R * BC * ESZ));
        const int nchunks = nblk * CPB;
        u32x4_t v[MAXC];
#pragma unroll
        for (int t = 0; t < MAXC; ++t) {
            const int c = threadIdx.x + t * NT;
            v[t] = __builtin_amdgcn_raw_buffer_load_b128(rA, c < nchunks ? c * 16 : (int)kOOB, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < MAXC; ++t) {
            const int c = threadIdx.x + t * NT;
            if (c < nchunks)
                *reinterpret_cast<u32x4_t *>(lds_a + (c / CPB) * ABUF + ((c % CPB) / CPR) * STRIDE +
                                             (c % CPR) * 16) = v[t];
        }
    }
    // block columns of the block row: lane q holds block q
    const __amdgpu_buffer_rsrc_t rJ = make_rsrc(p.col_idx + blk0, (uint32_t)nblk * 4u);
    const uint32_t vcols = __builtin_amdgcn_raw_buffer_load_b32(rJ, (uint32_t)lane * 4u, 0, 0);
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B, (uint32_t)p.b_bytes);
    const uint32_t ldb2 = (uint32_t)p.ldb * ESZ;   // bytes per B row
    const uint32_t k32 = (uint32_t)p.k;
    const uint32_t nbc = (uint32_t)((p.k + BC - 1) / BC);
    // this lane's first column in the first tile: row-major li*V + c, CM 16c + li
    const uint32_t lane_col = (uint32_t)(wave * 16 * V + (CM ? li : li * V));
    const int64_t col_first = t_begin * p.tile_cols + lane_col;
    const uint32_t tile_bytes = (uint32_t)p.tile_cols * ESZ;
    const int esz = p.c_dtype == SPMM_FP32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc((uint8_t *)p.C + row0 * p.ldc * esz, (uint32_t)(R * p.ldc * esz));
    // CM: one resource over the C^T rows this wave writes in the whole range
    const int64_t cm_n0 = t_begin * p.tile_cols + wave * 16 * V;
    const int64_t cm_n1 = (t_end - 1) * p.tile_cols + wave * 16 * V + 16 * V;
    const int64_t cm_end = cm_n1 < p.N ? cm_n1 : p.N;
    const uint32_t cm_size = CM && cm_end > cm_n0 ? (uint32_t)((cm_end - cm_n0) * p.ldc * esz) : 0u;
    const __amdgpu_buffer_rsrc_t rCt = make_rsrc((uint8_t *)p.C + (CM ? cm_n0 * p.ldc * esz : 0), cm_size);

    f32x4_t acc[MT][V];
    // B rows of half `half` of block q in tile t: J*64 + 32*half + 8g + j; tile
    // ntiles (past the range) loads nothing
    auto issue_b = [&](int t, int q, int half, BStage<DW> &st) {
        const uint32_t J = (uint32_t)__builtin_amdgcn_readlane((int)vcols, q);
        const bool jv = (t < ntiles) & (q < nblk) & (J < nbc);
        const uint32_t r0 = (jv ? J : 0u) * BC + (uint32_t)half * 32 + 8 * g;
        if constexpr (CM) {
            // the whole block as whole 128-byte lines: load e brings B^T rows
            // n_wave + 8e .. +7 (row n_wave + 8e + lane/8, the 16 bytes of k =
            // J*64 + 8*(lane%8) .. +7), eight rows per instruction instead of
            // sixteen half lines; compute_cm regroups them (`half` is unused)
            const uint32_t n0 = (uint32_t)(col_first - li) + (uint32_t)t * (uint32_t)p.tile_cols +
                                (uint32_t)(lane >> 3);
            const uint32_t kq = (jv ? J : 0u) * BC + 8 * (uint32_t)(lane & 7);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                buf_load<DW>(rB, (jv & (kq < k32)) ? (n0 + 8 * e) * ldb2 + kq * 2 : kOOB, st.b[e]);
        } else {
            const uint32_t base = r0 * ldb2 + (uint32_t)col_first * ESZ + (uint32_t)t * tile_bytes;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                buf_load<DW>(rB, (jv & (r0 + j < k32)) ? base + (uint32_t)j * ldb2 : kOOB, st.b[j]);
        }
    };
    auto compute = [&](const BStage<DW> &st, int q, int half) {
        if constexpr (F8) {
            // 8 fp8 codes of A per lane (8-byte LDS reads), B by byte transpose
            u32x2_t af[MT], bf[8];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[mt] = *reinterpret_cast<const u32x2_t *>(lds_a + q * ABUF + (mt * 16 + li) * STRIDE +
                                                           half * 32 + 8 * g);
            transpose8x8_bytes(st.b, bf);
#pragma unroll
            for (int c = 0; c < V; ++c)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][c] = mfma16x16x32_fp8(af[mt], bf[c], acc[mt][c]);
        } else {
        // row-major (column-major blocks go through compute_cm): lane group g of
        // half `half` holds k = 32*half + 8g .. +7
        u32x4_t af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            af[mt] = *reinterpret_cast<const u32x4_t *>(
                lds_a + q * ABUF + (mt * 16 + li) * STRIDE + (half * 32 + 8 * g) * 2);
#pragma unroll
        for (int c = 0; c < V; ++c) {
            u32x4_t bf;
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                bf[qq] = __builtin_amdgcn_perm(st.b[2 * qq + 1][c >> 1], st.b[2 * qq][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(af[mt], bf, acc[mt][c]);
        }
        }
    };
    // CM, one whole block: the eight loaded lines pass through the wave's
    // scratch 16 rows (one column group c) at a time, written with the 16-byte
    // chunk x of row r at slot x ^ (r % 8), so that the eight lanes of a read
    // phase hit eight different slots, and come back as MFMA operands: lane
    // (g, i) of half h reads chunk 4h + g of row i.  The scratch is private to
    // the wave and LDS instructions of a wave complete in order: no barrier.
    auto compute_cm = [&](const BStage<DW> &st, int q) {
        u32x4_t af[2][MT];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[hh][mt] = *reinterpret_cast<const u32x4_t *>(
                    lds_a + q * ABUF + (mt * 16 + li) * STRIDE + (hh * 32 + 8 * g) * 2);
#pragma unroll
        for (int c = 0; c < V; ++c) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                *reinterpret_cast<u32x4_t *>(scr + (8 * e + (lane >> 3)) * 128 +
                                             (((lane & 7) ^ (lane >> 3)) * 16)) =
                    u32x4_t{st.b[2 * c + e][0], st.b[2 * c + e][1], st.b[2 * c + e][2],
                            st.b[2 * c + e][3]};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4_t bf = *reinterpret_cast<const u32x4_t *>(
                    scr + li * 128 + (((4 * hh + g) ^ (li & 7)) * 16));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][c] = mfma16x16x32<AB>(af[hh][mt], bf, acc[mt][c]);
            }
        }
    };
    // stores tile t (one branch on C's type per tile)
    auto store_tile = [&](int t) {
        if constexpr (CM) {
            const uint32_t tile_off = (uint32_t)t * (uint32_t)p.tile_cols * (uint32_t)(p.ldc * esz);
            store_tile_cm(p.c_dtype, acc, rCt, cm_size, tile_off, g, li, row0, p.m, p.ldc);
        } else {
            const int64_t ncol = col_first + (int64_t)t * p.tile_cols;
            if (p.c_dtype == SPMM_FP32)
                store_acc_rows<SPMM_FP32>(acc, rC, g, row0, p.m, p.ldc, ncol, p.N);
            else if (p.c_dtype == SPMM_BF16)
                store_acc_rows<SPMM_BF16>(acc, rC, g, row0, p.m, p.ldc, ncol, p.N);
            else
                store_acc_rows<SPMM_FP16>(acc, rC, g, row0, p.m, p.ldc, ncol, p.N);
        }
    };
    auto zero_acc = [&]() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int c = 0; c < V; ++c)
                acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };

    if (nblk == 0) {  // empty block row: zero tiles
        zero_acc();
        for (int t = 0; t < ntiles; ++t)
            store_tile(t);
        return;
    }
    BStage<DW> st0, st1;
    issue_b(0, 0, 0, st0);
    if constexpr (CM) {
        // whole-block stages, two blocks per iteration: st0 holds block q, st1
        // block q + 1 (past the row's end, an odd count: zeros, not computed).
        // Every path issues the same loads, which keeps the wait counts exact.
        for (int t = 0; t < ntiles; ++t) {
            zero_acc();
            for (int q = 0; q < nblk; q += 2) {
                issue_b(t, q + 1, 0, st1);
                __builtin_amdgcn_sched_barrier(0);
                compute_cm(st0, q);
                __builtin_amdgcn_sched_barrier(0);
                const bool last = q + 2 >= nblk;
                issue_b(last ? t + 1 : t, last ? 0 : q + 2, 0, st0);
                __builtin_amdgcn_sched_barrier(0);
                if (q + 1 < nblk)
                    compute_cm(st1, q + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            store_tile(t);
        }
        return;
    }
    for (int t = 0; t < ntiles; ++t) {
        zero_acc();
        for (int q = 0; q < nblk; ++q) {
            // first half of block q (in st0): prefetch its second half
            issue_b(t, q, 1, st1);
            __builtin_amdgcn_sched_barrier(0);
            compute(st0, q, 0);
            __builtin_amdgcn_sched_barrier(0);
            // second half: prefetch the first half of the next block (or tile)
            const bool lastq = q + 1 == nblk;
            issue_b(lastq ? t + 1 : t, lastq ? 0 : q + 1, 0, st0);
            __builtin_amdgcn_sched_barrier(0);
            compute(st1, q, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        store_tile(t);
    }
}

// WCSR values into the tile kernel's A layout (see launch_wcsr_pack): one
// work-group per window, one 16-byte chunk per thread and turn.  Windows are
// b_col-padded, so the 8 entries of a chunk are all inside the window's width
// or all past it (zeros).
__global__ __launch_bounds__(256) void wcsr_pack_kernel(const uint16_t *__restrict__ values,
                                                        const int32_t *__restrict__ wptr,
                                                        const int32_t *__restrict__ pstart, int R,
                                                        uint16_t *__restrict__ out)
{
    const int64_t w = blockIdx.x;
    const uint32_t width = (uint32_t)(wptr[w + 1] - wptr[w]);
    const uint32_t steps = (width + 31u) / 32u;
    const uint32_t frags = (uint32_t)R / 16u;
    const uint32_t chunks = steps * frags * 64u;
    const __amdgpu_buffer_rsrc_t rV =
        make_rsrc(values + (int64_t)R * wptr[w], (uint32_t)R * width * 2u);
    uint16_t *const dst = out + (int64_t)R * pstart[w];
    for (uint32_t c = threadIdx.x; c < chunks; c += blockDim.x) {
        const uint32_t l = c & 63u, mt = (c >> 6) % frags, s = (c >> 6) / frags;
        const uint32_t row = 16u * mt + (l & 15u), col = 32u * s + 8u * (l >> 4);
        uint32_t v[4];
        buf_load<4>(rV, col < width ? (row * width + col) * 2u : kOOB, v);
        *reinterpret_cast<u32x4_t *>(dst + (int64_t)c * 8) = u32x4_t{v[0], v[1], v[2], v[3]};
    }
}

// BCSR 64x64 blocks into the fragment order (see launch_bcsr64_pack): one
// work-group per block, two 16-byte chunks per thread.
__global__ __launch_bounds__(256) void bcsr64_pack_kernel(const uint16_t *__restrict__ blocks,
                                                          uint16_t *__restrict__ out)
{
    const int64_t q = blockIdx.x;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(blocks + q * 4096, 8192u);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t c = threadIdx.x + 256u * t;
        const uint32_t l = c & 63u, hm = c >> 6;
        const uint32_t row = 16u * (hm % 4u) + (l & 15u), cc = 4u * (hm / 4u) + (l >> 4);
        uint32_t v[4];
        buf_load<4>(rA, (row * 64u + cc * 8u) * 2u, v);
        *reinterpret_cast<u32x4_t *>(out + q * 4096 + (int64_t)c * 8) = u32x4_t{v[0], v[1], v[2], v[3]};
    }
}

hipError_t launch_bcsr64_pack(const uint16_t *blocks, int64_t n_blocks, uint16_t *out, hipStream_t stream)
{
    if (n_blocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(bcsr64_pack_kernel, dim3((unsigned)n_blocks), dim3(256), 0, stream, blocks, out);
    return hipGetLastError();
}

hipError_t launch_wcsr_pack(const uint16_t *values, const int32_t *wptr, const int32_t *pstart,
                            int64_t n_windows, int R, uint16_t *out, hipStream_t stream)
{
    if (n_windows <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(wcsr_pack_kernel, dim3((unsigned)n_windows), dim3(256), 0, stream, values, wptr,
                       pstart, R, out);
    return hipGetLastError();
}

// Merge pass: one work-group per (merge record, 32 chunks of 8 tile columns).
// Eight adjacent lanes share a chunk: lane t adds slots t, t+8, t+16, ... in
// that order (its loads, two slots at a time, are independent of the other
// lanes'), then the eight running sums are combined pairwise across the lanes
// ((s0+s1)+(s2+s3))+((s4+s5)+(s6+s7)) and lane 0 writes C once.  The order
// depends only on the number of slots, so results are bitwise reproducible for
// a given plan, and a merge with up to 16 slots costs one memory round trip
// instead of one per four slots.
__global__ __launch_bounds__(256) void wcsr_merge_kernel(MergeParams p)
{
    const int3 mr = p.merges[blockIdx.x];
    const int t = threadIdx.x & 7;
    const int64_t chunk = (int64_t)blockIdx.y * 32 + (threadIdx.x >> 3);  // 8 columns each
    const int64_t per_row = p.N / 8;
    const int64_t r = chunk / per_row;
    const int64_t col = (chunk - r * per_row) * 8;
    const int64_t row = (int64_t)mr.x * p.R + r;
    const bool valid = (chunk < (int64_t)p.R * per_row) & (row < p.m);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float *src = p.partial + ((int64_t)mr.y * p.R + r) * p.N + col;
    const int64_t slot_stride = (int64_t)p.R * p.N;
    auto add = [&](const f32x4_t &a, const f32x4_t &b) {
        s[0] += a[0]; s[1] += a[1]; s[2] += a[2]; s[3] += a[3];
        s[4] += b[0]; s[5] += b[1]; s[6] += b[2]; s[7] += b[3];
    };
    if (valid) {
        int u = t;
        for (; u + 8 < mr.z; u += 16) {
            const float *q0 = src + u * slot_stride, *q1 = src + (u + 8) * slot_stride;
            const f32x4_t a0 = *reinterpret_cast<const f32x4_t *>(q0);
            const f32x4_t b0 = *reinterpret_cast<const f32x4_t *>(q0 + 4);
            const f32x4_t a1 = *reinterpret_cast<const f32x4_t *>(q1);
            const f32x4_t b1 = *reinterpret_cast<const f32x4_t *>(q1 + 4);
            add(a0, b0);
            add(a1, b1);
        }
        if (u < mr.z)
            add(*reinterpret_cast<const f32x4_t *>(src + u * slot_stride),
                *reinterpret_cast<const f32x4_t *>(src + u * slot_stride + 4));
    }
    // every lane of the wave takes part in the exchanges
#pragma unroll
    for (int off = 1; off < 8; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s[e] += __shfl_xor(s[e], off, 8);
    if (valid && t == 0)
        store_row<8>(p.C, row * p.ldc + col, p.c_dtype, s);
}

// The tile kernel instantiation for (format, tile rows, columns per lane, A/B type).
typedef void (*tile_fn_t)(TileParams);

template <int FMT, int R, int V>
static tile_fn_t tile_fn_ab(int ab)
{
    return ab == SPMM_FP16 ? spmm_tile_kernel<FMT, R, V, SPMM_FP16>
                           : spmm_tile_kernel<FMT, R, V, SPMM_BF16>;
}

// V = 8 exists for 16-row tiles only: taller tiles would need the ring's
// registers for their accumulators (the host never plans them).
template <int FMT, int R>
static tile_fn_t tile_fn_v(int v, int ab)
{
    if constexpr (R == 16)
        if (v == 8)
            return tile_fn_ab<FMT, R, 8>(ab);
    return v == 2 ? tile_fn_ab<FMT, R, 2>(ab) : v == 4 ? tile_fn_ab<FMT, R, 4>(ab) : nullptr;
}

template <int FMT>
static tile_fn_t tile_fn_r(int r, int v, int ab)
{
    return r == 16 ? tile_fn_v<FMT, 16>(v, ab) : r == 32 ? tile_fn_v<FMT, 32>(v, ab)
                                                         : tile_fn_v<FMT, 64>(v, ab);
}

static tile_fn_t tile_fn(int fmt, int R, int V, int ab)
{
    return fmt == 0 ? tile_fn_r<0>(R, V, ab) : tile_fn_r<1>(R, V, ab);
}

size_t tile_lds_bytes(int64_t buf_ints, int R, int V, int waves_n, int waves_k, bool two_buffers)
{
    const int64_t red = waves_k > 1 ? (int64_t)waves_n * waves_k * 4 * (R / 16) * V * 64 : 0;
    return (size_t)((two_buffers ? 2 : 1) * buf_ints + 256 + red) * sizeof(int32_t);
}

template <int NW, bool CM>
static void launch_lds_nw(int ab, const TileParams &p, hipStream_t stream)
{
    dim3 grid((unsigned)(p.n_items * p.n_col_tiles));
    if (ab == SPMM_FP16)
        hipLaunchKernelGGL((bcsr64_lds_kernel<SPMM_FP16, NW, CM>), grid, dim3(NW * 64), 0, stream,
                           p, p.col_idx);
    else
        hipLaunchKernelGGL((bcsr64_lds_kernel<SPMM_BF16, NW, CM>), grid, dim3(NW * 64), 0, stream,
                           p, p.col_idx);
}

hipError_t launch_bcsr64_lds(int ab, const TileParams &p, hipStream_t stream)
{
    if (p.col_major)
        p.waves_n == 1   ? launch_lds_nw<1, true>(ab, p, stream)
        : p.waves_n == 2 ? launch_lds_nw<2, true>(ab, p, stream)
        : p.waves_n == 8 ? launch_lds_nw<8, true>(ab, p, stream)
                         : launch_lds_nw<4, true>(ab, p, stream);
    else
        p.waves_n == 1   ? launch_lds_nw<1, false>(ab, p, stream)
        : p.waves_n == 2 ? launch_lds_nw<2, false>(ab, p, stream)
        : p.waves_n == 8 ? launch_lds_nw<8, false>(ab, p, stream)
                         : launch_lds_nw<4, false>(ab, p, stream);
    return hipGetLastError();
}

size_t sweep_lds_bytes(int max_blocks, int ab, bool col_major, int waves)
{
    return (size_t)(col_major ? waves * kSweepCmScratch : 0) +
           (size_t)max_blocks * 64 * (64 * (ab == SPMM_FP8_E4M3 ? 1 : 2) + 16);
}

static const void *sweep_fn(int ab, bool cm, int v, int waves)
{
    if (ab == SPMM_FP8_E4M3)
        return reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_FP8_E4M3, 4, false, 8>);
    if (cm && waves == 8)
        return ab == SPMM_FP16 ? reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_FP16, 8, true, 8>)
                               : reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_BF16, 8, true, 8>);
    if (cm)
        return ab == SPMM_FP16 ? reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_FP16, 4, true, 8>)
                               : reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_BF16, 4, true, 8>);
    if (v == 4)
        return ab == SPMM_FP16 ? reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_FP16, 4, false, 4>)
                               : reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_BF16, 4, false, 4>);
    return ab == SPMM_FP16 ? reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_FP16, 4, false, 8>)
                           : reinterpret_cast<const void *>(bcsr64_sweep_kernel<SPMM_BF16, 4, false, 8>);
}

hipError_t launch_bcsr64_sweep(int ab, int max_blocks, const TileParams &p, hipStream_t stream)
{
    TileParams arg = p;
    void *args[] = {&arg};
    const int waves = p.waves_n == 8 ? 8 : 4;
    return hipLaunchKernel(sweep_fn(ab, p.col_major != 0, p.tile_cols / (16 * waves), waves),
                           dim3((unsigned)(p.n_items * p.n_ranges)), dim3(64 * waves), args,
                           sweep_lds_bytes(max_blocks, ab, p.col_major != 0, waves), stream);
}

int sweep_blocks_per_cu(int ab, int max_blocks, bool col_major, int v, int waves)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, sweep_fn(ab, col_major, v, waves), 64 * waves,
                                                     sweep_lds_bytes(max_blocks, ab, col_major, waves)) != hipSuccess)
        return 0;
    return n;
}

hipError_t launch_tiles(int fmt, int R, int V, int ab, const TileParams &p, hipStream_t stream)
{
    if (!tile_fn(fmt, R, V, ab))
        return hipErrorInvalidValue;
    dim3 grid((unsigned)p.grid);
    dim3 block(64 * p.waves_n * p.waves_k);
    TileParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(tile_fn(fmt, R, V, ab)), grid, block,
                           args, tile_lds_bytes(p.lds_idx_ints, R, V, p.waves_n, p.waves_k, p.two_buffers != 0),
                           stream);
}

int tiles_blocks_per_cu(int fmt, int R, int V, int ab, int threads, size_t lds)
{
    int n = 0;
    const tile_fn_t f = tile_fn(fmt, R, V, ab);
    if (!f || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(f),
                                                           threads, lds) != hipSuccess)
        return 0;
    return n;
}

hipError_t launch_merge(const MergeParams &p, int64_t n_merges, hipStream_t stream)
{
    const int64_t chunks = (int64_t)p.R * (p.N / 8);
    dim3 grid((unsigned)n_merges, (unsigned)((chunks + 31) / 32));
    hipLaunchKernelGGL(wcsr_merge_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace wspmm

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
// a workspace slot; wcsr_merge adds the slots of a window in slot order and
// rounds once (this replaces the paper's atomicAdd merge, Section III-C).
//
// Work-group order: dispatch hands consecutive work-group ids to the 8 XCDs in
// turn.  The kernel renumbers ids so that each XCD receives a contiguous range
// of (column tile, work item) pairs, column tile outermost: the work-groups
// that share a column slice of B run on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace wspmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-class devices (no format conversion,
// no swizzle): the value the ROCm libraries use for gfx90a/gfx94x/gfx950.
constexpr int kRsrcWord3 = 0x00020000;
// Offset used for "no data": beyond any resource size the host allows.
constexpr uint32_t kOOB = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// Cache-policy bits of buffer instructions: non-temporal.  (Measured: on the
// generic kernel's A stream this is slower, the data then bypasses the MALL.)
constexpr int kNT = 2;

template <int DW, int POL = 0>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *out)
{
    if constexpr (DW == 4) {
        u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (DW == 2) {
        u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POL);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POL);
    }
}

template <int AB>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c)
{
    if constexpr (AB == SPMM_FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bfloat16 code, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> binary16 code (hardware conversion, round to nearest even).
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Stores V consecutive results of one row as c_dtype (NT: non-temporal stores).
template <typename T>
__device__ __forceinline__ void st(T *d, T x, bool nt)
{
    if (nt)
        __builtin_nontemporal_store(x, d);
    else
        *d = x;
}

template <int V, bool NT = false>
__device__ __forceinline__ void store_row(void *base, int64_t elem, int c_dtype, const float *v)
{
    if (c_dtype == SPMM_FP32) {
        float *d = reinterpret_cast<float *>(base) + elem;
        if constexpr (V >= 4) {
#pragma unroll
            for (int c = 0; c < V; c += 4)
                st(reinterpret_cast<f32x4_t *>(d + c), f32x4_t{v[c], v[c + 1], v[c + 2], v[c + 3]}, NT);
        } else {
            st(reinterpret_cast<f32x2_t *>(d), f32x2_t{v[0], v[1]}, NT);
        }
    } else {
        uint32_t w[V / 2];
#pragma unroll
        for (int c = 0; c < V; c += 2) {
            uint32_t lo = c_dtype == SPMM_BF16 ? f32_to_bf16(v[c]) : f32_to_f16(v[c]);
            uint32_t hi = c_dtype == SPMM_BF16 ? f32_to_bf16(v[c + 1]) : f32_to_f16(v[c + 1]);
            w[c / 2] = lo | (hi << 16);
        }
        uint16_t *d = reinterpret_cast<uint16_t *>(base) + elem;
        if constexpr (V == 8)
            st(reinterpret_cast<u32x4_t *>(d), u32x4_t{w[0], w[1], w[2], w[3]}, NT);
        else if constexpr (V == 4)
            st(reinterpret_cast<u32x2_t *>(d), u32x2_t{w[0], w[1]}, NT);
        else
            st(reinterpret_cast<uint32_t *>(d), w[0], NT);
    }
}

// Work-group id -> (work item, column tile), XCD-contiguous and column-tile major.
__device__ __forceinline__ void tile_of(int64_t n_items, int64_t total, int order, int64_t &item,
                                        int64_t &ctile)
{
    const int64_t i = blockIdx.x;
    const int64_t q = total >> 3, rem = total & 7;
    const int64_t xcd = i & 7, local = i >> 3;
    const int64_t logical = order ? i : xcd * q + (xcd < rem ? xcd : rem) + local;
    // (readfirstlane: tell the compiler these are wave-uniform, so that the
    // loads they address become scalar loads)
    ctile = __builtin_amdgcn_readfirstlane((int)(logical / n_items));
    item = __builtin_amdgcn_readfirstlane((int)(logical - ctile * n_items));
}

// Waits until this wave's LDS operations are done, then joins the work-group
// barrier.  Unlike __syncthreads() it does not wait for outstanding global
// loads, so prefetched B rows stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
    __builtin_amdgcn_s_barrier();
}

// One pipeline stage: the gathered B rows and the A fragments of one k' step.
template <int MT, int DW>
struct Stage {
    uint32_t b[8][DW];
    u32x4_t a[MT];
};

// Steps of B/A loads kept in flight ahead of the MFMAs (odd, so that the ring of
// D+1 register stages has an even size).  Chosen so that the ring, the
// accumulators and the addressing state fit about 240 VGPRs: two waves per SIMD.
template <int R, int V>
constexpr int pipe_depth()
{
    constexpr int acc = (R / 16) * V * 4;
    constexpr int stage = 8 * (V / 2) + (R / 16) * 4;
    constexpr int ring = (200 - acc) / stage;  // stages that fit
    return ring >= 4 ? 3 : 1;
}

// Generic tile kernel: one work-group per (task, column tile).  A task is a row
// tile (a BCSR block row or a WCSR window) and a range [kb0, kb1) of its packed
// columns; tasks that cover part of a row tile write an fp32 partial slot.
//   * The task's B-row indices (WCSR column indices, or BCSR block columns) are
//     copied into LDS once, so the main loop never waits on an index load queued
//     behind in-flight B loads.
//   * Each wave keeps D steps of A/B loads in flight in a ring of D+1 register
//     stages; all loads are issued unconditionally (steps past the end read
//     zeros), so the wait-count bookkeeping is the same on every path.
template <int FMT, int R, int V, int AB>
__global__ __launch_bounds__(256) void spmm_tile_kernel(TileParams p)
{
    constexpr int MT = R / 16;  // 16-row MFMA tiles per work-group tile
    constexpr int DW = V / 2;   // dwords of one gathered row segment per lane
    constexpr int D = pipe_depth<R, V>();
    constexpr int Q = D + 1;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int32_t *lidx = reinterpret_cast<int32_t *>(smem);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % p.waves_n;
    const int wk = wave / p.waves_n;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int nthreads = 64 * p.waves_n * p.waves_k;

    int64_t item, ctile;
    tile_of(p.n_items, p.n_items * p.n_col_tiles, p.order, item, ctile);

    // ---- task: row tile, packed-column range, A / index sources ------------
    const int4 t = p.tasks[item];
    const int64_t tile = t.x;
    const int32_t slot = t.w;
    const int64_t row0 = tile * R;
    const uint32_t klen = (uint32_t)(t.z - t.y);  // packed columns of the task
    const int64_t base = p.row_ptr[tile];
    const int64_t width = p.row_ptr[tile + 1] - base;  // WCSR window width
    const int32_t *gidx;
    uint32_t n_idx;              // index entries of the task
    __amdgpu_buffer_rsrc_t rA;
    uint32_t a_row_stride;       // bytes between A rows
    uint32_t a_col0;             // bytes to the task's first packed column in a row
    if constexpr (FMT == 0) {
        const int64_t blk0 = (int64_t)t.y >> p.log2_b_col;  // first block of the task
                                                             // (t.y counts from block 0)
        n_idx = klen >> p.log2_b_col;
        gidx = p.col_idx + blk0;
        rA = make_rsrc(p.A + blk0 * R * p.b_col, (uint32_t)((int64_t)n_idx * R * p.b_col * 2));
        a_row_stride = (uint32_t)p.b_col * 2;
        a_col0 = 0;
    } else {
        n_idx = klen;
        gidx = p.col_idx + t.y;
        rA = make_rsrc(p.A + R * base, (uint32_t)(R * width * 2));
        a_row_stride = (uint32_t)width * 2;
        a_col0 = (uint32_t)(t.y - base) * 2;
    }

    // ---- stage the task's indices in LDS (one burst per task) --------------
    // Direct-to-LDS buffer loads: each wave instruction fills a contiguous LDS run
    // (lane i -> bytes 16i or 4i); no VGPRs, one wait for the whole burst.
    {
        typedef __attribute__((address_space(3))) void lds_void;
        const __amdgpu_buffer_rsrc_t rI = make_rsrc(gidx, n_idx * 4);
        const int nwaves = p.waves_n * p.waves_k;
        if constexpr (FMT == 1) {
            // window column indices: n_idx is a multiple of 8, 16 bytes per lane
            for (int c = wave; c * 256 < (int)n_idx; c += nwaves)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rI, (lds_void *)(lidx + c * 256), 16,
                                                         (unsigned)((c * 64 + lane) * 16), 0, 0, 0);
        } else {
            // block columns: any count, 4 bytes per lane
            for (int c = wave; c * 64 < (int)n_idx; c += nwaves)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rI, (lds_void *)(lidx + c * 64), 4,
                                                         (unsigned)((c * 64 + lane) * 4), 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        lds_barrier();
    }
    // last valid start of an index read (reads past the task are masked anyway)
    const uint32_t idx_cap = (uint32_t)(p.lds_idx_ints > 8 ? p.lds_idx_ints - 8 : 0);

    // B resource starts at this wave's first column; rows are ldb apart.
    const int64_t col0 = ctile * p.tile_cols + wn * 16 * V;
    const uint64_t b_skip = (uint64_t)col0 * 2;
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(p.B + col0, (uint32_t)(p.b_bytes > b_skip ? p.b_bytes - b_skip : 0));
    const uint32_t ldb2 = (uint32_t)p.ldb * 2;
    const uint32_t lane_col_bytes = (uint32_t)li * V * 2;
    const uint32_t k32 = (uint32_t)p.k;
    const uint32_t nbc = (uint32_t)((p.k + p.b_col - 1) >> p.log2_b_col);  // block columns
    const int kspan = (int)klen - 32 * wk;
    const int nsteps = kspan > 0 ? (kspan + 32 * p.waves_k - 1) / (32 * p.waves_k) : 0;
    // this lane's first packed column (task-relative) at step s: kfirst + s * kstride
    const uint32_t kfirst = 32u * wk + 8u * g;
    const uint32_t kstride = 32u * p.waves_k;

    f32x4_t acc[MT][V];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < V; ++c)
            acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Issues the A and B loads of step s into st.
    auto issue = [&](int s, Stage<MT, DW> &st) {
        const uint32_t kl = kfirst + (uint32_t)s * kstride;  // task-relative packed column
        const bool ok = kl < klen;
        uint32_t a_off;
        if constexpr (FMT == 0) {
            const uint32_t q = kl >> p.log2_b_col;
            const uint32_t kk = kl & (uint32_t)(p.b_col - 1);
            const uint32_t J = (uint32_t)lidx[q < idx_cap ? q : idx_cap];  // in-bounds read
            const bool jv = ok & (J < nbc);
            const uint32_t r0 = (jv ? J : 0u) * (uint32_t)p.b_col + kk;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t r = r0 + j;
                buf_load<DW>(rB, (jv & (r < k32)) ? r * ldb2 + lane_col_bytes : kOOB, st.b[j]);
            }
            a_off = ((q * R + li) * (uint32_t)p.b_col + kk) * 2u;
        } else {
            const uint32_t kr = kl < idx_cap ? kl : idx_cap;  // in-bounds LDS read
            const u32x4_t i0 = *reinterpret_cast<const u32x4_t *>(lidx + kr);
            const u32x4_t i1 = *reinterpret_cast<const u32x4_t *>(lidx + kr + 4);
            const uint32_t ix[8] = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t r = ix[j];
                buf_load<DW>(rB, (ok & (r < k32)) ? r * ldb2 + lane_col_bytes : kOOB, st.b[j]);
            }
            a_off = li * a_row_stride + a_col0 + kl * 2u;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            uint32_t w[4];
            buf_load<4>(rA, ok ? a_off + (uint32_t)(mt * 16) * a_row_stride : kOOB, w);
            st.a[mt] = u32x4_t{w[0], w[1], w[2], w[3]};
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

    // ---- D-deep pipeline over the k' steps (nsteps is wave-uniform) --------
    if (nsteps > 0) {
        Stage<MT, DW> st[Q];
#pragma unroll
        for (int u = 0; u < D; ++u)
            issue(u, st[u]);
        for (int s = 0; s < nsteps; s += Q) {
#pragma unroll
            for (int u = 0; u < Q; ++u) {
                __builtin_amdgcn_sched_barrier(0);
                issue(s + u + D, st[(u + D) % Q]);
                __builtin_amdgcn_sched_barrier(0);
                compute(st[u]);  // steps past the end hold zeros: no branch in the ring
            }
        }
    }

    // ---- fixed-order sum of the waves_k partial tiles through LDS ----
    if (p.waves_k > 1) {
        constexpr int NR = MT * V * 4;
        float *red = reinterpret_cast<float *>(smem);  // [waves_n][NR][64], reuses the index area
        float *mine = red + (int64_t)wn * NR * 64 + lane;
        lds_barrier();  // every wave is done reading indices
        for (int s = p.waves_k - 1; s >= 1; --s) {
            if (wk == s) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int c = 0; c < V; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            mine[((mt * V + c) * 4 + q) * 64] = acc[mt][c][q];
            }
            lds_barrier();
            if (wk == 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int c = 0; c < V; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[mt][c][q] += mine[((mt * V + c) * 4 + q) * 64];
            }
            lds_barrier();
        }
        if (wk != 0)
            return;
    }

    // ---- epilogue: row 4g+q of each 16-row tile, V adjacent columns ----
    const int64_t ncol = col0 + li * V;
    if (ncol >= p.N)
        return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = mt * 16 + 4 * g + q;
            float v[V];
#pragma unroll
            for (int c = 0; c < V; ++c)
                v[c] = acc[mt][c][q];
            if (slot >= 0) {
                store_row<V>(p.partial, ((int64_t)slot * R + r) * p.N + ncol, SPMM_FP32, v);
            } else if (row0 + r < p.m) {
                store_row<V>(p.C, (row0 + r) * p.ldc + ncol, p.c_dtype, v);
            }
        }
    }
}

// BCSR with 64 x 64 blocks and a wide column tile (NW waves x 128 columns).
// Same MFMA mapping and B pipeline as spmm_tile_kernel, but the A block is
// shared: the work-group loads each 64 x 64 block once (non-temporal, it is
// streamed) into one of two padded LDS buffers, and every wave reads its A
// fragments from there.  Block-column indices are work-group uniform and come
// through scalar loads.  One LDS barrier per block.
template <int AB, int NW>
__global__ __launch_bounds__(NW * 64) void bcsr64_lds_kernel(TileParams p,
                                                             const int32_t *__restrict__ block_cols)
{
    constexpr int R = 64, BC = 64, MT = 4, V = 8, DW = 4;
    constexpr int NT = NW * 64;                    // threads per work-group
    constexpr int STRIDE = BC * 2 + 16;            // padded LDS row: conflict-free b128 reads
    constexpr int ABUF = R * STRIDE;               // bytes of one A buffer
    constexpr int CPT = R * BC / 8 / NT;           // 16-byte chunks per thread per block
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * ABUF];

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
    const uint64_t b_skip = (uint64_t)col0 * 2;
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(p.B + col0, (uint32_t)(p.b_bytes > b_skip ? p.b_bytes - b_skip : 0));
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

    // cooperative A-block copy: chunk c of a block = row c/8, 8 columns (c%8)*8
    auto load_a = [&](int q, u32x4_t (&r)[CPT]) {
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const int c = threadIdx.x + t * NT;
            r[t] = __builtin_amdgcn_raw_buffer_load_b128(
                rA, (int)(((uint32_t)q * R * BC + (uint32_t)c * 8) * 2), 0, kNT);
        }
    };
    auto store_a = [&](int buf, const u32x4_t (&r)[CPT]) {
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const int c = threadIdx.x + t * NT;
            *reinterpret_cast<u32x4_t *>(lds_a + buf * ABUF + (c >> 3) * STRIDE + (c & 7) * 16) =
                r[t];
        }
    };
    // Block column of block q (work-group uniform, so a scalar load); -1 past the end.
    auto block_col = [&](int q) -> uint32_t {
        const int at = __builtin_amdgcn_readfirstlane((int)blk0 + (q < nblk ? q : 0));
        const uint32_t J = (uint32_t)block_cols[at];
        return q < nblk ? J : 0xFFFFFFFFu;
    };
    // B rows of k' step s of block column J (half s%2): J*64 + 32*(s%2) + 8g + j
    auto issue_b = [&](int s, uint32_t J, Stage<MT, DW> &st) {
        const bool jv = J < nbc;
        const uint32_t r0 = (jv ? J : 0u) * BC + (uint32_t)(s & 1) * 32 + 8 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t r = r0 + j;
            buf_load<DW>(rB, (jv & (r < k32)) ? r * ldb2 + lane_col_bytes : kOOB, st.b[j]);
        }
    };
    auto compute = [&](const Stage<MT, DW> &st, int buf, int half) {
        u32x4_t af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            af[mt] = *reinterpret_cast<const u32x4_t *>(lds_a + buf * ABUF + (mt * 16 + li) * STRIDE +
                                                       (half * 32 + 8 * g) * 2);
#pragma unroll
        for (int c = 0; c < V; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t bf;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bf[q] = __builtin_amdgcn_perm(st.b[2 * q + 1][c >> 1], st.b[2 * q][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(af[mt], bf, acc[mt][c]);
        }
    };

    if (nblk > 0) {
        u32x4_t areg[CPT];
        Stage<MT, DW> st0, st1;
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

    // epilogue (non-temporal stores: C is written once)
    const int64_t ncol = col0 + li * V;
    if (ncol >= p.N)
        return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = mt * 16 + 4 * g + q;
            float v[V];
#pragma unroll
            for (int c = 0; c < V; ++c)
                v[c] = acc[mt][c][q];
            if (row0 + r < p.m)
                store_row<V, true>(p.C, (row0 + r) * p.ldc + ncol, p.c_dtype, v);
        }
    }
}

// One work-group per (merge record, chunk of 256*8 tile elements): adds the
// partial tiles of a split window in slot order and writes C once.
__global__ __launch_bounds__(256) void wcsr_merge_kernel(MergeParams p)
{
    const int3 mr = p.merges[blockIdx.x];
    const int64_t chunk = (int64_t)blockIdx.y * 256 + threadIdx.x;  // 8 columns each
    const int64_t per_row = p.N / 8;
    if (chunk >= (int64_t)p.R * per_row)
        return;
    const int64_t r = chunk / per_row;
    const int64_t col = (chunk - r * per_row) * 8;
    const int64_t row = (int64_t)mr.x * p.R + r;
    if (row >= p.m)
        return;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < mr.z; ++t) {
        const float *src = p.partial + ((int64_t)(mr.y + t) * p.R + r) * p.N + col;
        f32x4_t a = *reinterpret_cast<const f32x4_t *>(src);
        f32x4_t b = *reinterpret_cast<const f32x4_t *>(src + 4);
        s[0] += a[0]; s[1] += a[1]; s[2] += a[2]; s[3] += a[3];
        s[4] += b[0]; s[5] += b[1]; s[6] += b[2]; s[7] += b[3];
    }
    store_row<8>(p.C, row * p.ldc + col, p.c_dtype, s);
}

template <int FMT, int R, int V, int AB>
static hipError_t launch_one(const TileParams &p, dim3 grid, dim3 block, size_t lds,
                             hipStream_t stream)
{
    hipLaunchKernelGGL((spmm_tile_kernel<FMT, R, V, AB>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <int FMT, int R, int V>
static hipError_t by_ab(int ab, const TileParams &p, dim3 g, dim3 b, size_t lds, hipStream_t s)
{
    return ab == SPMM_FP16 ? launch_one<FMT, R, V, SPMM_FP16>(p, g, b, lds, s)
                           : launch_one<FMT, R, V, SPMM_BF16>(p, g, b, lds, s);
}

template <int FMT, int R>
static hipError_t by_v(int v, int ab, const TileParams &p, dim3 g, dim3 b, size_t lds,
                       hipStream_t s)
{
    switch (v) {
    case 2: return by_ab<FMT, R, 2>(ab, p, g, b, lds, s);
    case 4: return by_ab<FMT, R, 4>(ab, p, g, b, lds, s);
    default: return by_ab<FMT, R, 8>(ab, p, g, b, lds, s);
    }
}

template <int FMT>
static hipError_t by_r(int r, int v, int ab, const TileParams &p, dim3 g, dim3 b, size_t lds,
                       hipStream_t s)
{
    switch (r) {
    case 16: return by_v<FMT, 16>(v, ab, p, g, b, lds, s);
    case 32: return by_v<FMT, 32>(v, ab, p, g, b, lds, s);
    default: return by_v<FMT, 64>(v, ab, p, g, b, lds, s);
    }
}

size_t tile_lds_bytes(int R, int V, int waves_n, int waves_k, int64_t lds_idx_ints)
{
    const size_t red = waves_k > 1 ? (size_t)waves_n * (R / 16) * V * 4 * 64 * sizeof(float) : 0;
    const size_t idx = (size_t)lds_idx_ints * sizeof(int32_t);
    return red > idx ? red : idx;
}

template <int NW>
static void launch_lds_nw(int ab, const TileParams &p, hipStream_t stream)
{
    dim3 grid((unsigned)(p.n_items * p.n_col_tiles));
    if (ab == SPMM_FP16)
        hipLaunchKernelGGL((bcsr64_lds_kernel<SPMM_FP16, NW>), grid, dim3(NW * 64), 0, stream, p,
                           p.col_idx);
    else
        hipLaunchKernelGGL((bcsr64_lds_kernel<SPMM_BF16, NW>), grid, dim3(NW * 64), 0, stream, p,
                           p.col_idx);
}

hipError_t launch_bcsr64_lds(int ab, const TileParams &p, hipStream_t stream)
{
    if (p.waves_n == 2)
        launch_lds_nw<2>(ab, p, stream);
    else
        launch_lds_nw<4>(ab, p, stream);
    return hipGetLastError();
}

hipError_t launch_tiles(int fmt, int R, int V, int ab, const TileParams &p, hipStream_t stream)
{
    dim3 grid((unsigned)(p.n_items * p.n_col_tiles));
    dim3 block(64 * p.waves_n * p.waves_k);
    size_t lds = tile_lds_bytes(R, V, p.waves_n, p.waves_k, p.lds_idx_ints);
    return fmt == 0 ? by_r<0>(R, V, ab, p, grid, block, lds, stream)
                    : by_r<1>(R, V, ab, p, grid, block, lds, stream);
}

hipError_t launch_merge(const MergeParams &p, int64_t n_merges, hipStream_t stream)
{
    const int64_t chunks = (int64_t)p.R * (p.N / 8);
    dim3 grid((unsigned)n_merges, (unsigned)((chunks + 255) / 256));
    hipLaunchKernelGGL(wcsr_merge_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace wspmm

// Launch interface between the host API (api.hip) and the device kernels
// (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "window_spmm.h"

namespace wspmm {

// Arguments of the tile kernels.
struct TileParams {
    const uint16_t *A;        // BCSR blocks or WCSR window tiles (16-bit codes)
    const int32_t *col_idx;   // block_col_idx or window_col_idx
    const int32_t *row_ptr;   // block_row_ptr or window_row_ptr (plan-owned copy)
    const int32_t *tasks;     // generic kernel: work-item descriptors, 8 ints each:
                              // row tile, first packed column, end, slot (-1: writes C),
                              // WCSR window's first packed column, WCSR window width,
                              // column tile, 0
    const int32_t *lists;     // generic kernel: work-group b runs entries lists[b] .. lists[b+1]-1
    int64_t n_entries;        // generic kernel: descriptor table entries
    const uint16_t *B;        // k x N codes, leading dimension ldb
    int64_t ldb;
    void *C;                  // m x N of c_dtype, leading dimension ldc
    int64_t ldc;
    float *partial;           // partial tiles [slot][R][N] (fp32)
    int64_t m, k, N;
    uint64_t b_bytes;         // ((k - 1) * ldb + N) * 2: bytes of B the kernel may read
    int64_t n_items;          // tasks (generic kernel) or block rows (LDS-A kernel)
    int64_t n_col_tiles;      // column tiles; work items = n_items * n_col_tiles
    int64_t grid;             // generic kernel: persistent work-groups
    int32_t b_col;
    int32_t log2_b_col;       // BCSR: b_col is a power of two
    int32_t tile_cols;        // columns per work-group tile = waves_n * 16 * V
    int32_t waves_n;          // waves splitting the columns
    int32_t waves_k;          // waves splitting the packed-column reduction
    int32_t c_dtype;          // spmm_dtype_t of C
    int32_t order;            // LDS-A kernel: 0 XCD-contiguous, column-tile major; 1 launch order
    int32_t lds_idx_ints;     // generic kernel: ints of each LDS index buffer
    int32_t two_buffers;      // generic kernel: 0 if every work-group runs one entry (one buffer)
    int64_t n_ranges;         // sweep kernel: column ranges (a multiple of 8)
    int64_t range_tiles;      // sweep kernel: column tiles per range
    int32_t col_major;        // 64x64 kernels: B holds B^T (N rows of k), C holds C^T (N rows of m)
};

struct MergeParams {
    const int3 *merges;       // (window, first_slot, n_slots)
    const float *partial;     // [slot][R][N]
    void *C;
    int64_t ldc, m, N;
    int32_t R;
    int32_t c_dtype;
};

// Dynamic LDS bytes of the generic tile kernel: one or two index buffers of
// buf_ints ints, the sink and the cross-wave reduction area of its tile shape.
size_t tile_lds_bytes(int64_t buf_ints, int R, int V, int waves_n, int waves_k, bool two_buffers);

// Generic tile kernel, fmt: 0 = BCSR, 1 = WCSR; p.grid persistent work-groups.
hipError_t launch_tiles(int fmt, int R, int V, int ab_dtype, const TileParams &p, hipStream_t stream);
// Work-groups of the tile kernel <fmt, R, V, ab_dtype> resident per CU with
// `threads` threads and `lds_bytes` of dynamic LDS (0 if the query fails).
int tiles_blocks_per_cu(int fmt, int R, int V, int ab_dtype, int threads, size_t lds_bytes);
hipError_t launch_merge(const MergeParams &p, int64_t n_merges, hipStream_t stream);
// WCSR values -> the generic kernel's A layout.  Window w (packed columns
// [wptr[w], wptr[w+1]) of R-row tiles, each tile row-major R x W_w) becomes
// ceil(W_w / 32) steps of R x 32 entries at entry R * pstart[w], each step
// R / 16 fragments of 1 KB in MFMA operand order: the 16 bytes of lane
// l = 16g + i of fragment mt hold row 16mt + i, columns 32s + 8g .. +7 (zeros
// past W_w).  One work-group per window.
hipError_t launch_wcsr_pack(const uint16_t *values, const int32_t *wptr, const int32_t *pstart,
                            int64_t n_windows, int R, uint16_t *out, hipStream_t stream);
// BCSR 64x64 blocks -> the fragment order of the one-wave row-major form of
// bcsr64_lds_kernel: block q's 16-byte chunk c = (4h + mt) * 64 + 16g + i
// (row 16mt + i, columns 32h + 8g .. +7) at byte q * 8192 + 16c.  One
// work-group per block.
hipError_t launch_bcsr64_pack(const uint16_t *blocks, int64_t n_blocks, uint16_t *out, hipStream_t stream);
// BCSR with 64x64 blocks, waves_n (2 or 4) waves x 128 columns per work-group, A
// shared through LDS (requires waves_k = 1, V = 8, tile_cols = 128 * waves_n);
// p.col_major selects column-major B and C.
hipError_t launch_bcsr64_lds(int ab_dtype, const TileParams &p, hipStream_t stream);
// Most blocks in a block row that the sweep kernel holds in LDS.
constexpr int kSweepMaxBlocks = 8;
// Bytes of LDS per wave with which the sweep kernel regroups column-major B^T
// lines into MFMA operands (16 rows of 128 bytes; with 8 blocks of A a
// work-group then takes 80 KB, two per CU).
constexpr int kSweepCmScratch = 2048;
// BCSR with 64x64 blocks, A-stationary: n_items block rows x n_ranges column
// ranges of range_tiles tiles of p.tile_cols = 16 * (columns per lane) * waves columns
// (512 or 256; 256 with col_major and 4 waves), 4 waves (8 with col_major and
// p.waves_n = 8: 512-column tiles), every block of a block row in LDS
// (max_blocks <= kSweepMaxBlocks).
hipError_t launch_bcsr64_sweep(int ab_dtype, int max_blocks, const TileParams &p, hipStream_t stream);
// Dynamic LDS of one sweep work-group of `waves` waves: the CM scratch, then the A blocks.
size_t sweep_lds_bytes(int max_blocks, int ab_dtype, bool col_major, int waves);
// Work-groups of the sweep kernel resident per CU (0 if the query fails); waves
// per work-group 4, or 8 (column-major only, p.waves_n = 8).
int sweep_blocks_per_cu(int ab_dtype, int max_blocks, bool col_major, int cols_per_lane, int waves);
// Most blocks in a block row that the pair kernel holds in registers.
constexpr int kPairMaxBlocks = 6;
// BCSR with 64x64 blocks, A in the registers of a wave pair: n_items block rows x
// n_ranges column ranges of range_tiles strips of 128 columns (p.tile_cols =
// 128), two waves per work-group (FP16/BF16, row-major B and C).
hipError_t launch_bcsr64_pair(int ab_dtype, const TileParams &p, hipStream_t stream);
size_t pair_lds_bytes();
// Work-groups of the pair kernel resident per CU (0 if the query fails).
int pair_blocks_per_cu(int ab_dtype);
// Kernel 4: groups of kGroupRows block rows (64x64 blocks, at most kGroupMaxBlocks
// each) sharing B tiles through an LDS ring.  Group table (kGroupTableInts ints
// per group): rows[kGroupRows] (-1: none), nU, U[kGroupRows * kGroupMaxBlocks]
// (the union of the rows' block columns, increasing), cnt[same] (rows holding
// each union column), pos[kGroupRows][kGroupMaxBlocks] (union position of each
// row's q-th block).  p.n_items = groups, p.n_ranges ranges of p.range_tiles
// strips of 64 columns (p.tile_cols = 64).
constexpr int kGroupRows = 4;
constexpr int kGroupMaxBlocks = 6;
constexpr int kGroupTableInts = 80;
hipError_t launch_bcsr64_group(int ab_dtype, const TileParams &p, const int32_t *gtab,
                               hipStream_t stream);
size_t group_lds_bytes();
int group_blocks_per_cu(int ab_dtype);

}  // namespace wspmm

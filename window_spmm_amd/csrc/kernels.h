// Launch interface between the host API (api.hip) and the device kernels
// (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "window_spmm.h"

namespace wspmm {

// Arguments of the tile kernel (one work-group per (work item, column tile)).
struct TileParams {
    const uint16_t *A;        // BCSR blocks or WCSR window tiles (16-bit codes)
    const int32_t *col_idx;   // block_col_idx or window_col_idx
    const int32_t *row_ptr;   // block_row_ptr or window_row_ptr (plan-owned copy)
    const int4 *tasks;        // tasks (row tile, first packed column, end, slot); the BCSR
                              // LDS-A kernel walks whole block rows and ignores it
    const uint16_t *B;        // k x N codes, leading dimension ldb
    int64_t ldb;
    void *C;                  // m x N of c_dtype, leading dimension ldc
    int64_t ldc;
    float *partial;           // WCSR partial tiles [slot][R][N] (fp32)
    int64_t m, k, N;
    uint64_t b_bytes;         // k * ldb * 2: bytes of B the kernel may read (< 2^32 - 256)
    int64_t n_items;          // block rows (BCSR) or tasks (WCSR)
    int64_t n_col_tiles;      // column tiles; grid = n_items * n_col_tiles work-groups
    int32_t b_col;
    int32_t log2_b_col;       // BCSR: b_col is a power of two
    int32_t tile_cols;        // columns per work-group tile = waves_n * 16 * V
    int32_t waves_n;          // waves splitting the columns
    int32_t waves_k;          // waves splitting the packed-column reduction
    int32_t c_dtype;          // spmm_dtype_t of C
    int32_t order;            // 0: XCD-contiguous, column-tile major; 1: launch order
    int32_t lds_idx_ints;     // LDS index area (ints): every task's index count rounded up to
                              // 256, plus 256
};

struct MergeParams {
    const int3 *merges;       // (window, first_slot, n_slots)
    const float *partial;     // [slot][R][N]
    void *C;
    int64_t ldc, m, N;
    int32_t R;
    int32_t c_dtype;
};

// LDS bytes the tile kernel needs (task indices, reused for the cross-wave reduction).
size_t tile_lds_bytes(int R, int V, int waves_n, int waves_k, int64_t lds_idx_ints);

// fmt: 0 = BCSR, 1 = WCSR; work items are tasks in both (p.n_items of them).
hipError_t launch_tiles(int fmt, int R, int V, int ab_dtype, const TileParams &p, hipStream_t stream);
hipError_t launch_merge(const MergeParams &p, int64_t n_merges, hipStream_t stream);
// BCSR with 64x64 blocks, waves_n (2 or 4) waves x 128 columns per work-group, A
// shared through LDS (requires waves_k = 1, V = 8, tile_cols = 128 * waves_n).
hipError_t launch_bcsr64_lds(int ab_dtype, const TileParams &p, hipStream_t stream);

}  // namespace wspmm

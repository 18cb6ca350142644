/*
 * window_spmm — sparse x dense matrix multiply (SpMM) for AMD Instinct MI355X
 * (gfx950), in the two sparse formats of the AsyncSparse paper (Liu, Pu,
 * Zhang, "AsyncSparse: Accelerating Sparse Matrix-Matrix Multiplication on
 * Asynchronous GPU Architectures").
 *
 *   C[m x N] = A[m x k] * B[k x N]      A sparse, B and C dense, row-major.
 *
 * The operation is the one set up in the paper's Section II-C ("Sparse
 * Formats": A in R^{m x k} sparse, B in R^{k x n} dense, C = A x B).
 *
 * Conventions for every function below
 *  - Every function returns spmm_status_t and never throws or aborts.  On an
 *    error the outputs are unspecified, no plan is created, and
 *    spmm_last_error() returns a message for the calling thread.
 *  - Arguments prefixed h_ are host pointers, d_ are device pointers (memory
 *    of the current HIP device).  The caller owns every buffer it passes; the
 *    library never frees them.
 *  - Index arrays are int32; element offsets inside the library are 64-bit.
 *  - 16-bit values are passed as raw codes (uint16_t): IEEE binary16 or
 *    bfloat16 according to the dtype argument.  Builders copy codes bit-exactly.
 *  - Matrices are row-major; leading dimensions (ldb, ldc) count elements.
 *  - Test hook: with the environment variable SPMM_TEST_FAIL_ALLOC set to a
 *    value other than "" or "0", every host and device allocation the library
 *    makes fails, so that the SPMM_ERR_OUT_OF_MEMORY paths can be exercised.
 */
#ifndef WINDOW_SPMM_H
#define WINDOW_SPMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPMM_OK = 0,
    SPMM_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad block/window size */
    SPMM_ERR_BAD_FORMAT = 2,       /* inconsistent sparse arrays (see each function) */
    SPMM_ERR_UNSUPPORTED = 3,      /* valid input this build has no kernel for */
    SPMM_ERR_OUT_OF_MEMORY = 4,    /* host or device allocation failed */
    SPMM_ERR_HIP = 5               /* HIP runtime / launch error, or no usable gfx950 device */
} spmm_status_t;

/* Element types.  SPMM_FP8_E4M3: OCP FP8 E4M3 (1 sign, 4 exponent bits with
 * bias 7, 3 fraction bits, no infinities), the format of gfx950's fp8 MFMA;
 * A and B only (BCSR), the paper's first future direction (Section V). */
typedef enum { SPMM_FP16 = 0, SPMM_BF16 = 1, SPMM_FP32 = 2, SPMM_FP8_E4M3 = 3 } spmm_dtype_t;

typedef struct spmm_plan_s *spmm_plan_t;

/* Read-only description of a plan (for reports and tests). */
typedef struct {
    int32_t format;          /* 0 = BCSR, 1 = WCSR */
    int32_t tile_rows;       /* rows of C per work-group tile (= b_row) */
    int32_t tile_cols;       /* columns of C per work-group tile (BN) */
    int32_t waves_n;         /* waves splitting the tile's columns */
    int32_t waves_k;         /* waves splitting the reduction (packed columns) */
    int32_t cols_per_lane;   /* adjacent C columns each lane accumulates (V) */
    int32_t kernel;          /* 0: generic tile kernel; 1: BCSR 64x64 kernel with LDS-shared A;
                                2: BCSR 64x64 A-stationary sweep kernel;
                                3: BCSR 64x64 with A in the registers of a wave pair;
                                4: BCSR 64x64, groups of 4 block rows sharing B tiles */
    int32_t ranges_per_xcd;  /* kernels 2, 3, 4: column ranges per XCD (0 otherwise) */
    int32_t col_major;       /* 1 if the plan takes B^T and C^T (spmm_plan_options_t) */
    int32_t tuned;           /* configurations timed to choose this plan (0: not a tuned plan) */
    int64_t split_cols;      /* sub-task size T in packed columns (0: whole block rows) */
    int64_t n_tasks;         /* tasks (= work-groups per column tile; 0: whole block rows) */
    int64_t n_merges;        /* row tiles split into more than one task */
    int64_t n_slots;         /* partial-result slots in the workspace */
    int64_t stored_entries;  /* b_row*b_col*nnz_blocks (BCSR) or b_row*P (WCSR) */
    size_t workspace_bytes;  /* bytes of d_workspace spmm_*_run needs */
} spmm_plan_info_t;

/* ---------------------------------------------------------------------------
 * Host-side format builders (CPU only; no device needed).
 *
 * Input A is CSR: h_row_ptr[m+1] (non-decreasing, row_ptr[0] = 0), column
 * indices sorted strictly increasing inside each row and in [0, k), values as
 * 16-bit codes.  Every CSR entry is structural, whatever its value.
 * BAD_FORMAT: row_ptr not monotone / not starting at 0, a column out of range,
 * unsorted or duplicate columns in a row.  INVALID_ARGUMENT: m < 0, k < 0,
 * b_row or b_col outside [1, 1024], a required pointer null.
 * Each builder has a _count call that sizes the outputs, then a fill call.
 * ------------------------------------------------------------------------- */

/* BCSR (Section II-C "Block Compressed Sparse Row", Fig. 2): A is tiled into
 * b_row x b_col blocks; every block holding at least one entry is kept.
 * Outputs: block_row_ptr[ceil(m/b_row)+1], block_col_idx[nnz_blocks] (increasing
 * inside a block row), blocks[nnz_blocks*b_row*b_col]: each block a dense
 * row-major b_row x b_col tile, absent entries +0 (code 0x0000). */
spmm_status_t spmm_csr_to_bcsr_count(int64_t m, int64_t k, const int32_t *h_row_ptr,
                                     const int32_t *h_col_idx, int32_t b_row, int32_t b_col,
                                     int64_t *nnz_blocks);
spmm_status_t spmm_csr_to_bcsr(int64_t m, int64_t k, const int32_t *h_row_ptr,
                               const int32_t *h_col_idx, const uint16_t *h_values, int32_t b_row,
                               int32_t b_col, int32_t *h_block_row_ptr, int32_t *h_block_col_idx,
                               uint16_t *h_blocks);
/* The same for 8-bit codes (SPMM_FP8_E4M3 values): blocks[nnz_blocks*b_row*b_col]
 * bytes, absent entries 0x00 (+0). */
spmm_status_t spmm_csr_to_bcsr8(int64_t m, int64_t k, const int32_t *h_row_ptr,
                                const int32_t *h_col_idx, const uint8_t *h_values, int32_t b_row,
                                int32_t b_col, int32_t *h_block_row_ptr, int32_t *h_block_col_idx,
                                uint8_t *h_blocks);

/* WCSR (Section II-C "Window Compressed Sparse Row", Fig. 2): rows are grouped
 * into windows of b_row rows; window w keeps the sorted union of its rows'
 * column indices, padded with -1 up to the next multiple of b_col (W_w columns,
 * no extra group when the count divides evenly).  Outputs:
 * window_row_ptr[ceil(m/b_row)+1] (prefix sum of W_w; P = last entry),
 * window_col_idx[P], values[b_row*P]: window w's b_row x W_w tile is row-major
 * and starts at element b_row*window_row_ptr[w]; rows past m and pad columns
 * hold +0.  UNSUPPORTED if P >= 2^31. */
spmm_status_t spmm_csr_to_wcsr_count(int64_t m, int64_t k, const int32_t *h_row_ptr,
                                     const int32_t *h_col_idx, int32_t b_row, int32_t b_col,
                                     int64_t *padded_cols);
spmm_status_t spmm_csr_to_wcsr(int64_t m, int64_t k, const int32_t *h_row_ptr,
                               const int32_t *h_col_idx, const uint16_t *h_values, int32_t b_row,
                               int32_t b_col, int32_t *h_window_row_ptr, int32_t *h_window_col_idx,
                               uint16_t *h_values_out);

/* Window splitting (Section III-C: long windows become fixed-size sub-tasks and
 * each work-group takes one task descriptor).  A window of W <= split_cols
 * packed columns is one task (window, begin, end, -1) writing C directly; a
 * longer window becomes ceil(W/split_cols) tasks of split_cols columns (the last
 * one shorter) with consecutive partial slots, plus one merge record
 * (window, first_slot, n_slots).  Empty windows are one empty task.
 * tasks[n_tasks*4], merges[n_merges*3]; split_cols must be a positive multiple
 * of 32.  BAD_FORMAT if window_row_ptr is not monotone. */
spmm_status_t spmm_wcsr_split_count(int64_t n_windows, const int32_t *h_window_row_ptr,
                                    int64_t split_cols, int64_t *n_tasks, int64_t *n_merges);
spmm_status_t spmm_wcsr_split(int64_t n_windows, const int32_t *h_window_row_ptr,
                              int64_t split_cols, int32_t *h_tasks, int32_t *h_merges);

/* Reordering before the formats are built (Section IV-A: each evaluation
 * matrix is first reordered with reverse Cuthill-McKee, which clusters
 * nonzeros near the diagonal; Cuthill and McKee, "Reducing the bandwidth of
 * sparse symmetric matrices", 1969, with the numbering reversed).
 *
 * spmm_rcm_order: A is a square n x n CSR pattern (values not needed); the graph
 * is pattern(A) + pattern(A)^T without self loops.  h_perm[n] receives the
 * order: new position i holds old vertex h_perm[i].  The order is fixed by
 * these rules: components are numbered one after another, each starting from
 * the unplaced vertex of least degree (then least index), moved to a
 * pseudo-peripheral vertex by George and Liu's search (repeatedly root a level
 * structure at the least-degree, then least-index, vertex of the current last
 * level while that makes the structure taller); inside a component, vertices
 * are numbered breadth first and the unplaced neighbours of each vertex are
 * numbered by increasing degree, then index; finally the whole numbering is
 * reversed.  BAD_FORMAT / INVALID_ARGUMENT as for the builders;
 * UNSUPPORTED if n >= 2^31.
 *
 * spmm_csr_permute: the symmetric permutation A' = P A P^T of a square CSR
 * matrix: entry (h_perm[i], h_perm[j]) of A becomes entry (i, j) of A'.
 * Outputs h_out_row_ptr[n+1], h_out_col_idx[nnz], h_out_values[nnz] (columns
 * increasing in each row; codes copied bit-exactly).  With A' and B' = P B
 * (row i of B' = row h_perm[i] of B), C' = A' B' = P C: row i of C' is row
 * h_perm[i] of C.  INVALID_ARGUMENT if h_perm is not a permutation of 0..n-1. */
spmm_status_t spmm_rcm_order(int64_t n, const int32_t *h_row_ptr, const int32_t *h_col_idx,
                             int32_t *h_perm);
spmm_status_t spmm_csr_permute(int64_t n, const int32_t *h_row_ptr, const int32_t *h_col_idx,
                               const uint16_t *h_values, const int32_t *h_perm,
                               int32_t *h_out_row_ptr, int32_t *h_out_col_idx,
                               uint16_t *h_out_values);

/* ---------------------------------------------------------------------------
 * Plans.  A plan validates the format's host row pointer, picks the kernel
 * configuration for (format, b_row, b_col, N, dtypes), copies the small
 * metadata it needs to plan-owned device memory (block/window row pointer,
 * WCSR task and merge tables) and records the device pointers it is given.
 * Those device arrays (column indices, and the values) are read by every run
 * and must stay valid and unchanged until spmm_plan_destroy, except where the
 * plan copies the values into plan-owned memory (every WCSR plan, and a BCSR
 * plan on kernel 1 with one wave per work-group and row-major operands; see
 * spmm_wcsr_plan and spmm_bcsr_plan): its runs then read that copy, and later
 * writes to the values reach runs only through a new plan.  A plan is
 * immutable, so runs on different streams may overlap if each has its own
 * workspace and C.
 *
 * Supported: b_row in {16, 32, 64}; b_col a multiple of 8 (BCSR: a power of two
 * in [8, 256]);
 * ab_dtype FP16 or BF16 (A and B alike), or FP8_E4M3 for BCSR on kernel 2
 * (b_row = b_col = 64, N >= 4096, row-major B and C; values built with
 * spmm_csr_to_bcsr8, B one byte per element); c_dtype FP32, BF16 or FP16; N a
 * multiple of 8 (m = 0 or N = 0 gives a plan whose runs do nothing); k < 2^24
 * (B row numbers are multiplied in 24-bit arithmetic); device index and value
 * arrays 16-byte aligned.  Otherwise UNSUPPORTED.
 * Accumulation is fp32; 16-bit C is rounded once (nearest-even).
 * The plan needs a gfx950 device (SPMM_ERR_HIP otherwise).
 * *workspace_bytes receives the size of the workspace every run needs (0 if
 * none).
 * ------------------------------------------------------------------------- */

/* Plan options.  The kernel and tile shape are normally chosen by the plan;
 * these fields let a caller pin them, for a tile-width / wave-count sweep (the
 * measurement behind the paper's choice of tile width, Section IV-C, Fig. 7)
 * or to keep a configuration an autotuner found.  Each field's "auto" value
 * leaves that choice to the plan; spmm_plan_options_default() sets all of them.
 * A value outside its range is INVALID_ARGUMENT; a kernel that cannot run the
 * problem (see each kernel) is UNSUPPORTED. */
typedef struct {
    int32_t kernel;          /* -1 auto; 0 generic tile kernel (any format and shape);
                                1 BCSR 64x64 with LDS-shared A (b_row = b_col = 64; below
                                  N = 256 one wave per work-group, the plan's own choice
                                  from N = 128 with 16-bit row-major operands);
                                2 BCSR 64x64 A-stationary sweep (b_row = b_col = 64,
                                  N >= 4096, at most 8 blocks in every block row);
                                3 BCSR 64x64 with each block row's A in the registers of
                                  two waves, 128-column strips (b_row = b_col = 64,
                                  N >= 1024, at most 6 blocks in every block row, FP16 or
                                  BF16, row-major);
                                4 BCSR 64x64, block rows grouped four at a time by shared
                                  block columns, each group's B tiles staged once through
                                  an LDS ring and used by every row of the group that
                                  holds them (same limits as 3; 64-column strips, so
                                  cols_per_lane 0 or 4) */
    int32_t cols_per_lane;   /* 0 auto; kernel 0: 2, 4 or 8 adjacent C columns per lane
                                (8 only with b_row = 16); kernel 2: 8 (512-column tiles,
                                the default) or 4 (256-column tiles; FP16/BF16 only, and
                                the only choice with col_major) */
    int32_t waves_n;         /* 0 auto; kernel 0: 1, 2 or 4 waves across the tile's
                                columns; kernel 1: 1, 2, 4 or 8 waves of 128 columns (64
                                with col_major) (1: one wave per block row and tile, the
                                only form below N = 256 and the plan's choice there; 8 only
                                when pinned with kernel 1, or chosen by the plan at
                                N >= 8192); kernel 2 with col_major: 8
                                (pinned) for 8 waves of 64 columns, 512-column tiles,
                                instead of 4 (256-column tiles, the default) */
    int32_t waves_k;         /* 0 auto; kernel 0: 1, 2 or 4 waves splitting the packed
                                columns, waves_n * waves_k <= 4 */
    int32_t distribution;    /* -1 auto; kernel 0: 0 planned per-work-group task lists,
                                1 one work-group per task (hardware dispatch) */
    int32_t row_order;       /* -1 auto; kernel 0 with distribution 1: 0 longest task
                                first, 1 row order with a contiguous range per XCD */
    int32_t order;           /* -1 auto; kernel 1: 0 column-tile major with a contiguous
                                range per XCD (auto from N = 256), 1 launch order (auto
                                below N = 256) */
    int32_t ranges_per_xcd;  /* 0 auto; kernels 2, 3 and 4: column ranges per XCD, 1 to 64 */
    int32_t col_major;       /* 0: B is k x N and C is m x N, row-major (the default);
                                1: column-major, the layout of activations stored token by
                                token: d_B holds B^T (N rows of k, leading dimension ldb >= k)
                                and d_C holds C^T (N rows of m, ldc >= m).  BCSR with
                                b_row = b_col = 64, N >= 256, m and k multiples of 8, kernels 1
                                and 2 only (UNSUPPORTED otherwise); INVALID_ARGUMENT for WCSR. */
} spmm_plan_options_t;

void spmm_plan_options_default(spmm_plan_options_t *opt);

/* BCSR plan.  The product of the paper's BCSR kernel (Section III-A: each
 * work-group owns a block row and a column tile of C and walks the block row's
 * stored blocks, multiplying each dense block with the B tile of its block
 * column; Section IV-C: the tile width is chosen per N).
 * h_block_row_ptr[ceil(m/b_row)+1] (host, read during the call);
 * d_block_col_idx[nnz_blocks], d_blocks[nnz_blocks*b_row*b_col] (device; the
 * arrays spmm_csr_to_bcsr produced, copied to the device by the caller).
 * nnz_blocks is h_block_row_ptr[ceil(m/b_row)].
 * Block-column indices are read on the host only for a sample of up to 64
 * block rows (see "Synchronisation"); an index whose block lies outside
 * [0, k) contributes nothing (its B rows read as zero).  Long block rows
 * may be split into sub-tasks exactly like WCSR windows (same rule, counted in
 * packed columns = blocks * b_col) and merged in a fixed order; the plan then
 * needs a workspace.  UNSUPPORTED if nnz_blocks * b_col >= 2^31.
 * On kernel 1 with one wave per work-group and row-major B and C (the plan's
 * choice for b_row = b_col = 64 and 128 <= N < 256) the plan copies d_blocks
 * into plan-owned device memory (8 KB per block) in the order the kernel's
 * matrix instructions consume them (every A load of a run one contiguous 1 KB
 * run); the copy runs on the null stream and the plan waits for it (d_blocks
 * must be complete when the plan is called).
 * Synchronisation: a plan call is blocking.  It allocates and fills its device
 * tables with synchronous copies, and it reads a few device index entries back
 * to the host (synchronous device-to-host copies on the null stream, which
 * wait for the device) to tell banded from scattered patterns.  Make plans
 * outside timed or captured regions. */
spmm_status_t spmm_bcsr_plan(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N, int32_t b_row,
                             int32_t b_col, const int32_t *h_block_row_ptr,
                             const int32_t *d_block_col_idx, const void *d_blocks,
                             spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype, size_t *workspace_bytes);
/* The same with options (NULL: all automatic, as spmm_bcsr_plan). */
spmm_status_t spmm_bcsr_plan_ex(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N, int32_t b_row,
                                int32_t b_col, const int32_t *h_block_row_ptr,
                                const int32_t *d_block_col_idx, const void *d_blocks,
                                spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                const spmm_plan_options_t *options, size_t *workspace_bytes);

/* WCSR plan.  The product of the paper's WCSR kernel (Section III-B and
 * Section III-C: a work-group gathers the B rows named by its window's column
 * union and multiplies them with the window's packed value tile; long windows
 * are cut into fixed-size sub-tasks, one task descriptor per work-group, whose
 * partial tiles are merged -- here by a second pass in a fixed order instead of
 * the paper's atomic adds).
 * h_window_row_ptr[ceil(m/b_row)+1] (host; every window width a
 * multiple of b_col, else BAD_FORMAT); d_window_col_idx[P], d_values[b_row*P]
 * (device), P = h_window_row_ptr[ceil(m/b_row)].  A column index outside
 * [0, k) (the -1 pads included) reads B as zero.  split_cols: sub-task size T
 * (positive multiple of 32, at most 8192), or 0 to let the plan choose.
 * UNSUPPORTED if a window tile (b_row * width * 2 bytes) reaches 2^32 - 256.
 * The plan copies d_values into plan-owned device memory in the order the
 * kernel's matrix instructions consume them (each window's width rounded up to
 * a multiple of 32 with zeros: b_row * P' * 2 bytes, P' <= P + 24 per window;
 * every A load of a run is then one contiguous 1 KB run); the copy runs on the
 * null stream and the plan waits for it, so d_values must be complete when the
 * plan is called (writes on a non-blocking stream synchronised first).  Writes to d_values after the plan
 * call reach runs only through a new plan.  OUT_OF_MEMORY if the copy cannot
 * be allocated.  Synchronisation otherwise as for spmm_bcsr_plan. */
spmm_status_t spmm_wcsr_plan(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N, int32_t b_row,
                             int32_t b_col, const int32_t *h_window_row_ptr,
                             const int32_t *d_window_col_idx, const void *d_values,
                             spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype, int64_t split_cols,
                             size_t *workspace_bytes);
/* The same with options (NULL: all automatic, as spmm_wcsr_plan); kernel must
 * be -1 or 0. */
spmm_status_t spmm_wcsr_plan_ex(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N, int32_t b_row,
                                int32_t b_col, const int32_t *h_window_row_ptr,
                                const int32_t *d_window_col_idx, const void *d_values,
                                spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype, int64_t split_cols,
                                const spmm_plan_options_t *options, size_t *workspace_bytes);

/* Tuned plans.  The paper measures throughput against the tile width and keeps
 * the best (Section IV-C, Fig. 7); the plans above choose with fixed rules from
 * the problem's shape instead.  A tuned plan makes that measurement on the
 * caller's operands: it makes the plan spmm_*_plan_ex would make with `options`,
 * then a plan for every configuration from a fixed candidate list that keeps
 * the fields `options` pins (the 64x64 block kernels with their range and tile
 * variants, the generic kernel's columns per lane, wave splits and task
 * distribution; for WCSR with split_cols = 0 also sub-task sizes 128, 512, 2048
 * and 8192), times each on `stream` (two untimed runs, then `reps` runs between
 * two events; reps = 0: about 4 ms of runs, at least 5 and at most 100), then
 * times the four fastest three more times each, interleaved with the automatic
 * plan, and returns the one with the lowest median if it is at least 2 % faster
 * than the automatic plan's median (else the automatic plan; the sub-task sizes
 * are a second such stage after the first).  Candidates no kernel can run,
 * and candidates whose plan or workspace cannot be allocated beside the plans
 * held (at most six at a time, each with its tables and any value copy), are
 * skipped.  Arguments as for
 * spmm_*_plan_ex, plus the operands of the runs to time: d_B, ldb, d_C, ldc as
 * for spmm_*_run (the same requirements, checked before anything is launched).
 * d_C is overwritten: on return it holds the product from one of the timed
 * plans; run the returned plan for the result.  chosen (may be NULL) receives
 * the options the returned plan was made with (fields left automatic stay so;
 * spmm_plan_info gives what the plan picked for them, and tuned = the number of
 * configurations timed).  The call is blocking (it waits for the timed runs)
 * and allocates a workspace for the candidates that need one, freed before it
 * returns.  INVALID_ARGUMENT if reps is outside [0, 10000]; errors of the
 * automatic plan or of a launch are returned as such. */
spmm_status_t spmm_bcsr_plan_tuned(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                   int32_t b_row, int32_t b_col, const int32_t *h_block_row_ptr,
                                   const int32_t *d_block_col_idx, const void *d_blocks,
                                   spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                   const spmm_plan_options_t *options, const void *d_B, int64_t ldb,
                                   void *d_C, int64_t ldc, void *stream, int32_t reps,
                                   spmm_plan_options_t *chosen, size_t *workspace_bytes);
spmm_status_t spmm_wcsr_plan_tuned(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                   int32_t b_row, int32_t b_col, const int32_t *h_window_row_ptr,
                                   const int32_t *d_window_col_idx, const void *d_values,
                                   spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype, int64_t split_cols,
                                   const spmm_plan_options_t *options, const void *d_B, int64_t ldb,
                                   void *d_C, int64_t ldc, void *stream, int32_t reps,
                                   spmm_plan_options_t *chosen, size_t *workspace_bytes);

/* Run: C = A * B (the problem of Section II-C: A sparse m x k, B dense k x N),
 * computed by the kernels of Section III-A..III-C as chosen by the plan, fp32
 * accumulation, one rounding to c_dtype.  Enqueued on `stream` (a hipStream_t;
 * NULL = the null stream), no host synchronisation and no allocation.  d_B: k x N codes with leading dimension ldb (the
 * kernels read no byte past element (k - 1) * ldb + N - 1); d_C:
 * m x N of c_dtype with leading dimension ldc.  Rows < m and columns < N of C
 * are overwritten (C is never read); rows without entries become 0.
 * Requirements (else UNSUPPORTED): d_B and d_C 16-byte aligned, ldb >= N and
 * ldc >= N, both multiples of 8, ldb < 2^23, k * ldb * 2 < 2^32 - 256 and
 * b_row * ldc * (C element bytes) < 2^32 - 256 (B and a tile's rows of C are
 * addressed through 32-bit buffer offsets).  A plan made with col_major = 1
 * takes d_B = B^T (N rows of k, ldb >= k) and d_C = C^T (N rows of m, ldc >= m):
 * ldb, ldc multiples of 8, ldb < 2^23, N * ldb * 2 and (N + 1024) * ldc * (C
 * element bytes) below 2^32 - 256; the kernels read no byte of B^T past element
 * (N - 1) * ldb + k - 1.  d_workspace: at least workspace_bytes of
 * device memory (16-byte aligned) when workspace_bytes > 0, else ignored.
 * Device-side faults surface at the caller's next synchronisation. */
spmm_status_t spmm_bcsr_run(spmm_plan_t plan, const void *d_B, int64_t ldb, void *d_C, int64_t ldc,
                            void *d_workspace, void *stream);
spmm_status_t spmm_wcsr_run(spmm_plan_t plan, const void *d_B, int64_t ldb, void *d_C, int64_t ldc,
                            void *d_workspace, void *stream);

/* The WCSR run for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and result as spmm_wcsr_run, but the fp32 partial tiles of split
 * windows go into a static device array of the library,
 * SPMM_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, instead of a workspace.  The call
 * allocates and frees nothing; the caller still passes B and C as for
 * spmm_wcsr_run, with the same requirements.  UNSUPPORTED if the plan's
 * workspace_bytes exceeds SPMM_NOALLOC_SCRATCH_BYTES (a larger split size
 * shrinks it).  Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams, or a run still executing) race and
 * give wrong results; serialise them or use spmm_wcsr_run with a workspace each.
 * The array keeps the last call's contents; nothing needs clearing (every
 * partial slot a run reads is written earlier in the same run).  The first call
 * on a device looks up the array's address on that device. */
#define SPMM_NOALLOC_SCRATCH_BYTES (32u << 20)
spmm_status_t spmm_wcsr_run_noalloc(spmm_plan_t plan, const void *d_B, int64_t ldb, void *d_C,
                                    int64_t ldc, void *stream);

spmm_status_t spmm_plan_info(spmm_plan_t plan, spmm_plan_info_t *info);

/* Leading dimension (elements) to allocate for a dense operand with N columns of
 * elem_bytes-byte elements: N rounded up to 8; when that row pitch is a multiple
 * of 4 KiB, plus 2 KiB of elements (1024 for 2-byte, 2048 for 1-byte, 512 for
 * 4-byte elements) if the pitch is 16 KiB or more, else plus 64 elements (128
 * for 1-byte elements).  With a 4 KiB-multiple pitch, the rows that one column
 * tile reads all fall into the same L2 sets; from 16 KiB on, a pitch half a page
 * past the multiple also makes a run's time independent of where B and C were
 * allocated.  Any ldb/ldc >= N that is a multiple of 8 is valid; this only
 * affects speed.  Returns N unchanged for N <= 0 or elem_bytes <= 0. */
int64_t spmm_recommended_ld(int64_t N, int32_t elem_bytes);

/* Launch floor: enqueues one empty kernel (one work-group of 64 threads) on
 * `stream` (a hipStream_t; NULL = the null stream).  A measurement aid: timed
 * like a run, it gives the cost of a launch that does no work, against which
 * the runs of small problems are read.  SPMM_ERR_HIP if the launch fails
 * (e.g. no device). */
spmm_status_t spmm_launch_floor(void *stream);

/* Frees the plan's host and device memory.  NULL is accepted.  The caller must
 * make sure no run using the plan is still executing. */
spmm_status_t spmm_plan_destroy(spmm_plan_t plan);

const char *spmm_status_string(spmm_status_t status);
/* Message describing the calling thread's last error ("" if none). */
const char *spmm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WINDOW_SPMM_H */

// C-ABI entry points: plans and runs for BCSR and WCSR SpMM on gfx950.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <functional>
#include <cstring>
#include <mutex>
#include <new>
#include <queue>
#include <vector>

#include "common.h"
#include "kernels.h"

struct spmm_plan_s {
    int fmt;                    // 0 = BCSR, 1 = WCSR
    int64_t m, k, N;
    int32_t b_row, b_col;
    int ab, ct;
    const uint16_t *A;          // BCSR: the caller's blocks; WCSR: d_apack
    const int32_t *col_idx;
    uint16_t *d_apack;          // plan-owned copy of the values in fragment order: WCSR
                                // (launch_wcsr_pack), BCSR on the one-wave row-major
                                // LDS-A kernel (launch_bcsr64_pack)
    const std::vector<int32_t> *h_pstart;  // WCSR, while planning: first packed entry / b_row
                                           // of each window in d_apack
    int32_t *d_row_ptr;         // plan-owned copy of the block / window row pointer
    int32_t *d_tasks;           // work-item descriptors, 8 ints each (TileParams::tasks)
    int32_t *d_lists;           // per-work-group ranges of d_tasks (TileParams::lists)
    bool two_buffers;           // work-groups run several entries (TileParams::two_buffers)
    int64_t n_entries;          // entries of d_tasks
    int32_t *d_merges;          // (row tile, first_slot, n_slots)
    int32_t *d_groups;          // kernel 4: group tables (kGroupTableInts ints each)
    int64_t n_items;            // work items per column tile: block rows (LDS kernel)
                                // or task-table entries, padding included (tile kernel)
    int64_t n_tasks;            // tasks without the padding
    int order;                  // work-group -> item mapping (TileParams::order)
    int64_t n_merges, n_slots, split_cols;
    int64_t lds_idx_ints;       // ints of each LDS index buffer of the generic kernel
    int64_t grid;               // persistent work-groups of the generic kernel
    int64_t stored_entries;
    int V, waves_n, waves_k;
    int kernel;                 // 0: generic tile kernel, 1: BCSR 64x64 with LDS-shared A,
                                // 2: BCSR 64x64, A-stationary sweep over column ranges,
                                // 3: BCSR 64x64, A in the registers of a wave pair
    int max_blocks;             // kernel 2: most blocks in a block row (LDS size)
    spmm_plan_options_t opt;    // the caller's choices (auto fields: the plan's)
    int64_t n_ranges, range_tiles;  // kernels 2, 3: column ranges (multiple of 8), tiles each
    int64_t tile_cols, n_col_tiles;
    size_t workspace;
    int device;
    int n_tuned;                // configurations timed to choose this plan (0: not tuned)
};

namespace wspmm {
namespace {

// Buffer resources address at most 2^32 bytes; the kernels use offsets above
// this bound as "read zero".
constexpr uint64_t kMaxBBytes = 0xFFFFFF00ull;

// Range checks of plan options that do not depend on the matrix.
spmm_status_t check_options(const spmm_plan_options_t &o, bool bcsr)
{
    if (o.kernel < -1 || o.kernel > 4 || (!bcsr && o.kernel > 0))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "options.kernel %d is not a kernel of this format",
                    o.kernel);
    if (o.cols_per_lane != 0 && o.cols_per_lane != 2 && o.cols_per_lane != 4 && o.cols_per_lane != 8)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "options.cols_per_lane must be 0, 2, 4 or 8");
    // waves_n 8: the LDS-A kernel's 8-wave tiles (kernel 1 pinned), or the sweep
    // kernel's column-major 8-wave tiles (kernel 2 pinned, col_major)
    const bool lds8 = (o.kernel == 1 || (o.kernel == 2 && o.col_major == 1)) && o.waves_n == 8 &&
                      o.waves_k == 0;
    if (!lds8 && (o.waves_n < 0 || o.waves_n > 4 || o.waves_n == 3 || o.waves_k < 0 || o.waves_k > 4 ||
                  o.waves_k == 3 || std::max(1, o.waves_n) * std::max(1, o.waves_k) > 4))
        return fail(SPMM_ERR_INVALID_ARGUMENT,
                    "options.waves_n and waves_k must be 0, 1, 2 or 4 with a product of at most 4 "
                    "(waves_n 8 only with kernel 1, or kernel 2 with col_major)");
    if (o.distribution < -1 || o.distribution > 1 || o.row_order < -1 || o.row_order > 1 ||
        o.order < -1 || o.order > 1)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "options.distribution, row_order and order must be -1, 0 or 1");
    if (o.ranges_per_xcd < 0 || o.ranges_per_xcd > 64)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "options.ranges_per_xcd must be in [0, 64]");
    if (o.col_major < 0 || o.col_major > 1 || (!bcsr && o.col_major))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "options.col_major must be 0 or 1 (0 for WCSR)");
    return SPMM_OK;
}

spmm_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(SPMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The library only runs on gfx950; find out whether the current device is one.
spmm_status_t current_device(int *dev, int *n_cu, int64_t *lds_per_cu, int64_t *l2_bytes)
{
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count == 0)
        return fail(SPMM_ERR_HIP, "no HIP device available");
    if ((e = hipGetDevice(dev)) != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, *dev)) != hipSuccess)
        return hip_fail(e, "hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(SPMM_ERR_HIP, "device %d is %s, this library is built for gfx950", *dev,
                    prop.gcnArchName);
    *n_cu = prop.multiProcessorCount;
    *lds_per_cu = (int64_t)prop.maxSharedMemoryPerMultiProcessor;
    *l2_bytes = (int64_t)prop.l2CacheSize;
    return SPMM_OK;
}

spmm_status_t check_common(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N, int32_t b_row,
                           int32_t b_col, const int32_t *h_ptr, const void *d_idx,
                           const void *d_vals, spmm_dtype_t ab, spmm_dtype_t ct,
                           size_t *workspace_bytes, bool bcsr)
{
    if (!plan || !workspace_bytes || !h_ptr)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null plan, workspace_bytes or row pointer");
    if (m < 0 || k < 0 || N < 0)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "negative size");
    if (b_row < 1 || b_col < 1)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "block/window size must be positive");
    if (b_row != 16 && b_row != 32 && b_row != 64)
        return fail(SPMM_ERR_UNSUPPORTED, "b_row = %d: supported 16, 32, 64", b_row);
    if (b_col % 8 != 0 || (bcsr && (b_col > 256 || (b_col & (b_col - 1)) != 0)))
        return fail(SPMM_ERR_UNSUPPORTED, "b_col = %d: must be %s", b_col,
                    bcsr ? "a power of two in [8, 256]" : "a multiple of 8");
    if (ab != SPMM_FP16 && ab != SPMM_BF16 && !(bcsr && ab == SPMM_FP8_E4M3))
        return fail(SPMM_ERR_UNSUPPORTED, "A/B dtype must be FP16 or BF16 (FP8_E4M3: BCSR only)");
    if (ct != SPMM_FP32 && ct != SPMM_BF16 && ct != SPMM_FP16)
        return fail(SPMM_ERR_UNSUPPORTED, "C dtype must be FP32, BF16 or FP16");
    if (N % 8 != 0)
        return fail(SPMM_ERR_UNSUPPORTED, "N = %lld must be a multiple of 8", (long long)N);
    if (N > (int64_t(1) << 28) || m >= (int64_t(1) << 31) || k >= (int64_t(1) << 31))
        return fail(SPMM_ERR_UNSUPPORTED, "matrix dimension too large");
    if (k >= (int64_t(1) << 24))
        return fail(SPMM_ERR_UNSUPPORTED, "k = %lld: must be below 2^24", (long long)k);
    if (((uintptr_t)d_idx | (uintptr_t)d_vals) & 15)
        return fail(SPMM_ERR_UNSUPPORTED, "device index/value arrays must be 16-byte aligned");
    const int64_t nrow = ceil_div(m, b_row);
    if (h_ptr[0] != 0)
        return fail(SPMM_ERR_BAD_FORMAT, "row pointer must start at 0");
    for (int64_t i = 0; i < nrow; ++i) {
        if (h_ptr[i + 1] < h_ptr[i])
            return fail(SPMM_ERR_BAD_FORMAT, "row pointer decreases at %lld", (long long)i);
        if (!bcsr && (h_ptr[i + 1] - h_ptr[i]) % b_col != 0)
            return fail(SPMM_ERR_BAD_FORMAT, "window %lld width is not a multiple of b_col",
                        (long long)i);
    }
    if (h_ptr[nrow] > 0 && (!d_idx || !d_vals))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null device index or value array");
    return SPMM_OK;
}

// Tile shape: V columns per lane (wave width 16V), waves along N, waves along k'.
// wide: 16-row tiles take two waves along N when N spans two or more wave
// widths, so that one work-group covers 256 columns and each window's indices
// and values are read once (used for row-ordered plans with few items).
spmm_status_t choose_config(spmm_plan_s *pl, double mean_kprime, int n_cu, bool wide)
{
    const spmm_plan_options_t &o = pl->opt;
    int V = pl->N >= 128 ? 8 : (pl->N >= 64 ? 4 : 2);
    if (pl->b_row >= 32 && V > 4)
        V = 4;  // taller tiles: the accumulators at V = 8 leave no room for the ring
                // (the kernel has no such instantiation)
    if (o.cols_per_lane > 0) {
        if (pl->b_row >= 32 && o.cols_per_lane > 4)
            return fail(SPMM_ERR_UNSUPPORTED, "8 columns per lane need b_row = 16");
        V = o.cols_per_lane;
    }
    const int64_t wave_cols = 16 * V;
    const int64_t col_waves = ceil_div(pl->N, wave_cols);
    int wn = o.waves_n > 0 ? o.waves_n
             : (pl->b_row == 64 && col_waves >= 2) ? 2
             : (wide && pl->b_row == 16 && col_waves >= 2) ? 2 : 1;
    const int64_t col_tiles = std::max<int64_t>(1, ceil_div(pl->N, wave_cols * wn));
    // add reduction waves while the grid is small (below 12 waves per CU) and
    // the items are long (every wave keeps at least 4 steps of 32 packed
    // columns per item).  Measured on the WCSR population: small uniform
    // matrices with 2500-4000 windows of 130-280 packed columns ran 10-25 %
    // faster with one reduction wave than with the two a 16-waves-per-CU,
    // 2-steps-per-wave rule gave them; the 16384^2 WCSR workload (1024 windows
    // of 2066 columns on average) keeps its 4.
    const int64_t waves = std::max<int64_t>(1, pl->n_items * col_tiles * wn);
    int wk = 1;
    while (wn * wk * 2 <= 4 && waves * wk < int64_t(12) * n_cu && mean_kprime >= 128.0 * wk * 2)
        wk *= 2;
    if (o.waves_k > 0)
        wk = o.waves_k;
    if (wn * wk > 4)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "waves_n * waves_k must be at most 4");
    pl->V = V;
    pl->waves_n = wn;
    pl->waves_k = wk;
    pl->tile_cols = wave_cols * wn;
    pl->n_col_tiles = pl->N > 0 ? ceil_div(pl->N, pl->tile_cols) : 0;
    return SPMM_OK;
}

template <typename T>
spmm_status_t upload(const T *h, int64_t n, T **d)
{
    *d = nullptr;
    if (n == 0)
        return SPMM_OK;
    if (test_fail_alloc())
        return fail(SPMM_ERR_OUT_OF_MEMORY, "device allocation of %lld bytes refused "
                    "(SPMM_TEST_FAIL_ALLOC)", (long long)(sizeof(T) * n));
    hipError_t e = hipMalloc(reinterpret_cast<void **>(d), sizeof(T) * (size_t)n);
    if (e != hipSuccess) {
        *d = nullptr;
        return fail(SPMM_ERR_OUT_OF_MEMORY, "hipMalloc of %lld bytes failed: %s",
                    (long long)(sizeof(T) * n), hipGetErrorString(e));
    }
    e = hipMemcpy(*d, h, sizeof(T) * (size_t)n, hipMemcpyHostToDevice);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpy");
    return SPMM_OK;
}

void free_plan(spmm_plan_s *pl)
{
    if (!pl)
        return;
    if (pl->d_row_ptr) (void)hipFree(pl->d_row_ptr);
    if (pl->d_tasks) (void)hipFree(pl->d_tasks);
    if (pl->d_lists) (void)hipFree(pl->d_lists);
    if (pl->d_merges) (void)hipFree(pl->d_merges);
    if (pl->d_groups) (void)hipFree(pl->d_groups);
    if (pl->d_apack) (void)hipFree(pl->d_apack);
    delete pl;
}

spmm_status_t check_run(spmm_plan_t pl, const void *B, int64_t ldb, void *C, int64_t ldc,
                        void *ws)
{
    if (!pl)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null plan");
    if (pl->m == 0 || pl->N == 0)
        return SPMM_OK;
    if (!C || (pl->k > 0 && !B))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null B or C");
    if (((uintptr_t)B | (uintptr_t)C) & 15)
        return fail(SPMM_ERR_UNSUPPORTED, "B and C must be 16-byte aligned");
    const bool cm = pl->opt.col_major != 0;
    const uint64_t esz = pl->ct == SPMM_FP32 ? 4u : 2u;
    const uint64_t esz_b = pl->ab == SPMM_FP8_E4M3 ? 1u : 2u;
    if (cm ? (ldb < pl->k || ldc < pl->m) : (ldb < pl->N || ldc < pl->N))
        return fail(SPMM_ERR_UNSUPPORTED, cm ? "column-major: ldb must be >= k and ldc >= m"
                                             : "ldb/ldc must be >= N");
    if (ldb % 8 || ldc % 8)
        return fail(SPMM_ERR_UNSUPPORTED, "ldb/ldc must be multiples of 8");
    if (ldb >= (int64_t(1) << 23))
        return fail(SPMM_ERR_UNSUPPORTED, "ldb must be below 2^23");
    if ((uint64_t)(cm ? pl->N : pl->k) * (uint64_t)ldb * esz_b >= kMaxBBytes)
        return fail(SPMM_ERR_UNSUPPORTED, "B must be smaller than 4 GiB - 256 bytes");
    // (the last column tile's lanes address up to 511 columns past N; their
    // 32-bit store offsets must stay past the end of C^T without wrapping)
    if (cm && (uint64_t)(pl->N + 1024) * (uint64_t)ldc * esz >= kMaxBBytes)
        return fail(SPMM_ERR_UNSUPPORTED, "C^T ((N + 1024) * ldc * element bytes) must be below 4 GiB - 256");
    if ((uint64_t)pl->b_row * (uint64_t)ldc * (pl->ct == SPMM_FP32 ? 4u : 2u) >= kMaxBBytes)
        return fail(SPMM_ERR_UNSUPPORTED, "b_row rows of C (b_row * ldc * element bytes) must be below 4 GiB");
    if (pl->workspace > 0 && (!ws || ((uintptr_t)ws & 15)))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "plan needs a 16-byte aligned workspace of %zu bytes",
                    pl->workspace);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != pl->device)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "plan was made on device %d, current is %d",
                    pl->device, dev);
    return SPMM_OK;
}

spmm_status_t run_plan(spmm_plan_t pl, int fmt, const void *B, int64_t ldb, void *C, int64_t ldc,
                       void *ws, void *stream)
{
    spmm_status_t s = check_run(pl, B, ldb, C, ldc, ws);
    if (s != SPMM_OK)
        return s;
    if (pl->fmt != fmt)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "plan format does not match the run call");
    if (pl->m == 0 || pl->N == 0 || pl->n_items == 0)
        return ok();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    TileParams p;
    p.A = pl->A;
    p.col_idx = pl->col_idx;
    p.row_ptr = pl->d_row_ptr;
    p.tasks = pl->d_tasks;
    p.lists = pl->d_lists;
    p.two_buffers = pl->two_buffers ? 1 : 0;
    p.n_entries = pl->n_entries;
    p.B = reinterpret_cast<const uint16_t *>(B);
    p.ldb = ldb;
    p.C = C;
    p.ldc = ldc;
    p.partial = reinterpret_cast<float *>(ws);
    p.m = pl->m;
    p.k = pl->k;
    p.N = pl->N;
    // the extent of B ends with column N - 1 of row k - 1: loads of columns past N
    // in that row and of rows past k fall outside it and read zeros
    const uint64_t esz_b = pl->ab == SPMM_FP8_E4M3 ? 1u : 2u;
    p.b_bytes = pl->opt.col_major
                    ? ((uint64_t)(pl->N - 1) * (uint64_t)ldb + (uint64_t)pl->k) * esz_b
                    : pl->k > 0 ? ((uint64_t)(pl->k - 1) * (uint64_t)ldb + (uint64_t)pl->N) * esz_b : 0u;
    p.col_major = pl->opt.col_major;
    p.n_items = pl->n_items;
    p.n_col_tiles = pl->n_col_tiles;
    p.b_col = pl->b_col;
    p.log2_b_col = 0;
    while ((1 << p.log2_b_col) < pl->b_col)
        ++p.log2_b_col;
    p.tile_cols = (int32_t)pl->tile_cols;
    p.waves_n = pl->waves_n;
    p.waves_k = pl->waves_k;
    p.c_dtype = pl->ct;
    p.order = pl->order;
    p.lds_idx_ints = (int32_t)pl->lds_idx_ints;
    p.grid = pl->grid;
    p.n_ranges = pl->n_ranges;
    p.range_tiles = pl->range_tiles;
    hipError_t e = pl->kernel == 4   ? launch_bcsr64_group(pl->ab, p, pl->d_groups, st)
                   : pl->kernel == 3 ? launch_bcsr64_pair(pl->ab, p, st)
                   : pl->kernel == 2 ? launch_bcsr64_sweep(pl->ab, pl->max_blocks, p, st)
                   : pl->kernel == 1 ? launch_bcsr64_lds(pl->ab, p, st)
                                     : launch_tiles(fmt, pl->b_row, pl->V, pl->ab, p, st);
    if (e != hipSuccess)
        return hip_fail(e, "tile kernel launch");
    if (pl->n_merges > 0) {
        MergeParams mp;
        mp.merges = reinterpret_cast<const int3 *>(pl->d_merges);
        mp.partial = reinterpret_cast<const float *>(ws);
        mp.C = C;
        mp.ldc = ldc;
        mp.m = pl->m;
        mp.N = pl->N;
        mp.R = pl->b_row;
        mp.c_dtype = pl->ct;
        e = launch_merge(mp, pl->n_merges, st);
        if (e != hipSuccess)
            return hip_fail(e, "merge kernel launch");
    }
    return ok();
}

}  // namespace
}  // namespace wspmm

using namespace wspmm;

namespace wspmm {
namespace {

// Sub-task size when the caller leaves it to the plan.  `slots` work-groups of
// the tile kernel are resident at once.  If no row tile is longer than
// `slack10` tenths of the total work divided by the slots, T covers the longest
// one (nothing is cut, no merge pass); otherwise T is that quotient, so that no
// task outlasts the average work of a slot.  T is a multiple of `align`, at
// least 512 and at most kMaxSplit.
constexpr int64_t kMaxSplit = 8192;
// slack10 of persistent plans.  Their work-groups share CUs in pairs and the
// assignment is balanced with the longest tasks first, so a task up to half as
// long again as a slot's share still ends with its CU; a merge pass costs a
// launch and a round trip (measured on the 16384^2 WCSR workload: its longest
// window, 1.32 shares, cut into tasks and merged ran 51.2-51.5 us, uncut
// 49.0-49.4 us).
constexpr int64_t kPersistentSlack10 = 15;

int64_t auto_split(int64_t n_rows, const std::function<int64_t(int64_t)> &start, int64_t align,
                   int64_t slots, int64_t slack10)
{
    const int64_t total = start(n_rows) - start(0);
    int64_t longest = 0;
    for (int64_t w = 0; w < n_rows; ++w)
        longest = std::max(longest, start(w + 1) - start(w));
    const int64_t share = ceil_div(total, std::max<int64_t>(1, slots));
    int64_t T = longest * 10 <= share * slack10 ? longest : share;
    T = std::max<int64_t>(512, ceil_div(T, align) * align);
    return std::min<int64_t>(T, kMaxSplit);
}

// Work of an item for the assignment: its packed columns plus a fixed share
// for the per-task start-up and finish.
constexpr int64_t kTaskOverhead = 512;
// Work-groups g and g + n_cu share a CU (dispatch fills every CU once before
// any twice).  Where two share a SIMD the waves of the later one issue after
// those of the earlier one; measured on the WCSR and BCSR workloads, the later
// work-group then progresses about 1.6 to 1.8 times slower, so the assignment
// charges its work at this factor (in tenths).
constexpr int64_t kLateSlotCost10 = 16;
// Items per resident work-group from which every item gets a work-group of its
// own and the hardware dispatcher balances the load (the real cost of a task
// also depends on how its B rows hit the caches, which a static plan does not
// see; with few items per work-group the static plan, whose work-groups
// overlap one task's start with the previous task, is better).
constexpr int64_t kSpreadItems = 6;

// Splits the row tiles into tasks (row tile w covers packed columns
// [start(w), start(w+1))), sizes the two LDS index buffers (`shift`: log2 of
// packed columns per index entry; they also hold the cross-wave reduction) and
// the workspace, sets the persistent grid, and assigns the work items (task,
// column tile) to the work-groups: longest first, each to the least loaded
// work-group (ties: lowest index), a work-group running its items in the order
// they were assigned.  Uploads the descriptor table (work-group major), the
// per-work-group ranges and the merge table.
spmm_status_t make_tasks(spmm_plan_s *pl, int64_t n_rows, const std::function<int64_t(int64_t)> &start,
                         int64_t split_cols, int shift, int n_cu, bool spread, bool local)
{
    try {
        alloc_probe();
        std::vector<int32_t> tasks, merges;
        split_tasks(n_rows, start, split_cols, tasks, merges);
        const int64_t nt = (int64_t)tasks.size() / 4, nm = (int64_t)merges.size() / 3;
        int64_t slots = 0, max_idx = 0;
        for (int64_t i = 0; i < nm; ++i)
            slots += merges[3 * i + 2];
        for (int64_t i = 0; i < nt; ++i)
            max_idx = std::max<int64_t>(max_idx, (int64_t)(tasks[4 * i + 2] - tasks[4 * i + 1]) >> shift);
        pl->n_tasks = nt;
        pl->n_items = nt;
        pl->n_merges = nm;
        pl->n_slots = slots;
        pl->split_cols = split_cols;
        // index copies write whole 256-int runs; reads start at most 8 before the end
        pl->lds_idx_ints = ceil_div(max_idx, 256) * 256 + 256;
        pl->two_buffers = !spread;
        const size_t lds = tile_lds_bytes(pl->lds_idx_ints, pl->b_row, pl->V, pl->waves_n, pl->waves_k,
                                          pl->two_buffers);
        const int per_cu = tiles_blocks_per_cu(pl->fmt, pl->b_row, pl->V, pl->ab,
                                               64 * pl->waves_n * pl->waves_k, lds);
        if (per_cu < 1)
            return fail(SPMM_ERR_HIP, "tile kernel cannot be resident (LDS %zu bytes)", lds);
        const int64_t n_work = nt * pl->n_col_tiles;
        // spread: one work-group per item, in longest-first order
        const int64_t G = spread ? std::max<int64_t>(1, n_work)
                                 : std::max<int64_t>(1, std::min<int64_t>(n_work, (int64_t)n_cu * per_cu));

        // Greedy longest-first assignment.  Work-group g runs on XCD g mod 8
        // (dispatch is round-robin over the XCDs), so with several column
        // tiles the items of one column tile go to the work-groups of a fixed
        // subset of XCDs: each XCD's L2 then holds only its column slices of B.
        const int64_t n_ct = pl->n_col_tiles;
        const int64_t groups =
            (n_ct > 1 && n_ct <= 8 && 8 % n_ct == 0) ? n_ct : (n_ct > 8 && n_ct % 8 == 0) ? 8 : 1;
        const int64_t xcd_groups = groups;
        std::vector<int64_t> order(n_work);
        for (int64_t i = 0; i < n_work; ++i)
            order[i] = i;
        const auto cost = [&](int64_t item) {
            const int64_t t = item % std::max<int64_t>(1, nt);
            return (int64_t)tasks[4 * t + 2] - tasks[4 * t + 1] + kTaskOverhead;
        };
        if (spread && local) {
            // Row order, each XCD a contiguous range (work-group g runs on XCD
            // g mod 8): B is much larger than an L2, and neighbouring row tiles
            // of banded patterns gather the same B rows.
            const int64_t q = n_work / 8, rem = n_work % 8;
            for (int64_t g = 0; g < n_work; ++g) {
                const int64_t x = g % 8, l = g / 8;
                order[g] = x * q + std::min(x, rem) + l;
            }
        } else {
            std::stable_sort(order.begin(), order.end(),
                             [&](int64_t a, int64_t b) { return cost(a) > cost(b); });
        }
        // SIMD-sharing level of work-group g: 0 for the first waves on each SIMD
        const int waves_wg = pl->waves_n * pl->waves_k;
        const int64_t late10 = kLateSlotCost10;
        const auto weight10 = [&](int64_t g) -> int64_t {
            return ((g / n_cu) * waves_wg) / 4 > 0 ? late10 : 10;
        };
        typedef std::pair<int64_t, int64_t> load_t;  // (load in tenths, work-group)
        typedef std::priority_queue<load_t, std::vector<load_t>, std::greater<load_t>> heap_t;
        std::vector<heap_t> heap(xcd_groups);
        for (int64_t g = 0; g < G; ++g)
            heap[(g % 8) % xcd_groups].push({0, g});
        for (auto &h : heap)
            if (h.empty())
                return fail(SPMM_ERR_UNSUPPORTED, "grid of %lld work-groups too small", (long long)G);
        std::vector<int64_t> owner(n_work), count(G + 1, 0);
        for (int64_t i = 0; i < n_work; ++i) {
            if (spread) {
                owner[i] = i;
                ++count[i + 1];
                continue;
            }
            heap_t &h = heap[(order[i] / std::max<int64_t>(1, nt)) % xcd_groups];
            load_t l = h.top();
            h.pop();
            owner[i] = l.second;
            ++count[l.second + 1];
            h.push({l.first + cost(order[i]) * weight10(l.second), l.second});
        }
        std::vector<int32_t> lists(G + 1, 0);
        for (int64_t g = 0; g < G; ++g)
            lists[g + 1] = (int32_t)(lists[g] + count[g + 1]);
        std::vector<int32_t> fill(lists.begin(), lists.end() - 1);
        std::vector<int32_t> desc(8 * n_work, 0);
        for (int64_t i = 0; i < n_work; ++i) {
            const int64_t item = order[i], t = item % nt;
            const int32_t *src = &tasks[4 * t];
            int32_t *d = &desc[8 * (int64_t)fill[owner[i]]++];
            std::copy_n(src, 4, d);
            if (pl->fmt == 1) {
                d[4] = (int32_t)start(src[0]);
                d[5] = (int32_t)(start(src[0] + 1) - start(src[0]));
                d[7] = pl->h_pstart ? (*pl->h_pstart)[src[0]] : 0;
            }
            d[6] = (int32_t)(item / nt);  // column tile
        }
        pl->grid = G;
        pl->n_entries = n_work;
        spmm_status_t s;
        if ((s = upload(desc.data(), n_work * 8, &pl->d_tasks)) != SPMM_OK ||
            (s = upload(lists.data(), G + 1, &pl->d_lists)) != SPMM_OK ||
            (s = upload(merges.data(), nm * 3, &pl->d_merges)) != SPMM_OK)
            return s;
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    if (pl->n_merges > 0 && ceil_div((int64_t)pl->b_row * (pl->N / 8), 32) > 65535)
        return fail(SPMM_ERR_UNSUPPORTED, "N too large for the merge grid");
    if (pl->n_merges > 0 && (uint64_t)pl->b_row * (uint64_t)pl->N * 4u >= kMaxBBytes)
        return fail(SPMM_ERR_UNSUPPORTED, "b_row * N * 4 bytes of a partial tile must be below 4 GiB");
    pl->workspace = (size_t)pl->n_slots * (size_t)pl->b_row * (size_t)pl->N * sizeof(float);
    return SPMM_OK;
}

// Whether the pattern is banded: the median column span (last minus first
// column) of up to 64 row tiles spread over the matrix is below k/8.  Reads
// the first index and the last b_col indices (WCSR pads with -1 at the end) of
// each sampled tile from the device.  `ptr` is the host row pointer, `idx` the
// device index array, `unit` the columns per index (b_col for BCSR, 1 for WCSR).
bool banded_pattern(int64_t n_rows, const int32_t *ptr, const int32_t *idx, int64_t unit, int64_t k,
                    int64_t tail)
{
    std::vector<int64_t> spans;
    const int64_t samples = std::min<int64_t>(64, n_rows);
    for (int64_t i = 0; i < samples; ++i) {
        const int64_t w = (2 * i + 1) * n_rows / (2 * samples);
        const int64_t a = ptr[w], b = ptr[w + 1];
        if (b <= a)
            continue;
        int32_t lo = 0;
        std::vector<int32_t> hi((size_t)std::min<int64_t>(tail, b - a));
        if (hipMemcpy(&lo, idx + a, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(hi.data(), idx + b - (int64_t)hi.size(), hi.size() * sizeof(int32_t),
                      hipMemcpyDeviceToHost) != hipSuccess)
            return false;
        int32_t top = lo;
        for (int32_t v : hi)
            top = std::max(top, v);
        spans.push_back((int64_t)(top - lo) * unit);
    }
    if (spans.empty())
        return false;
    std::nth_element(spans.begin(), spans.begin() + spans.size() / 2, spans.end());
    return spans[spans.size() / 2] * 8 < k;
}

// Tile shape, split size and work assignment of the tile kernel for row tiles
// whose packed columns are [start(w), start(w+1)).  split_cols = 0: chosen here.
spmm_status_t plan_tasks(spmm_plan_s *pl, int64_t n_rows, const std::function<int64_t(int64_t)> &start,
                         int64_t split_cols, int64_t align, int shift, int n_cu, int64_t lds_per_cu,
                         int64_t l2_bytes, const int32_t *h_ptr)
{
    const int64_t total = start(n_rows) - start(0);
    pl->n_items = n_rows;
    // A banded pattern whose B is much larger than an L2: one work-group per
    // item, in row order with a contiguous range of rows per XCD, so that
    // neighbouring row tiles share B rows in that XCD's L2.  Where that is what
    // turns the plan from lists into one work-group per item (few items), the
    // tile also takes 256 columns.  Measured on the WCSR population's banded
    // members at N = 256 against longest-first lists: 35232 rows 88.0 -> 52.5
    // us, 54803 rows 212.5 -> 100.3 us; at 343589 to 400511 rows, which have
    // items enough for one work-group each anyway, 128-column tiles stay
    // 9-19 % faster.
    const bool banded_large =
        pl->k * pl->N * 2 > 2 * std::max<int64_t>(1, l2_bytes) &&
        banded_pattern(n_rows, h_ptr, pl->col_idx, pl->fmt == 0 ? pl->b_col : 1, pl->k,
                       pl->fmt == 0 ? 1 : pl->b_col);
    const bool want_local = pl->opt.distribution != 0 && pl->opt.row_order != 0 && banded_large;
    const double mean_kprime = n_rows > 0 ? (double)total / (double)n_rows : 0.0;
    int64_t slots = 0;
    int per_cu_regs = 1;
    size_t lds0 = 0;
    bool many = false;
    for (int pass = 0; pass < 2; ++pass) {
        spmm_status_t s = choose_config(pl, mean_kprime, n_cu, pass == 1);
        if (s != SPMM_OK)
            return s;
        const int threads = 64 * pl->waves_n * pl->waves_k;
        // work-groups per CU that registers allow
        lds0 = tile_lds_bytes(0, pl->b_row, pl->V, pl->waves_n, pl->waves_k, true);
        per_cu_regs = std::max(1, tiles_blocks_per_cu(pl->fmt, pl->b_row, pl->V, pl->ab, threads, lds0));
        slots = (int64_t)n_cu * per_cu_regs;
        if (pass == 0)
            many = n_rows * pl->n_col_tiles >= kSpreadItems * slots;
        if (!want_local || many)
            break;
    }
    const bool spread = pl->opt.distribution >= 0 ? pl->opt.distribution == 1 : want_local || many;
    if (split_cols == 0) {
        // the index buffers of every resident work-group must fit its share of
        // the LDS, which caps the task length
        const int64_t buf_max = ((lds_per_cu / per_cu_regs - (int64_t)lds0) / 4) / (spread ? 1 : 2);
        int64_t cap = ((buf_max - 256) / 256 * 256) << shift;
        cap = std::max<int64_t>(512, cap / align * align);
        split_cols = auto_split(n_rows, start, align, slots / std::max<int64_t>(1, pl->n_col_tiles),
                                spread ? 10 : kPersistentSlack10);
        split_cols = std::min(split_cols, std::max<int64_t>(align, cap));
    }
    // Spread work-groups run in row order when B is much larger than an L2 and
    // the pattern is banded (neighbouring row tiles then share B rows);
    // otherwise longest first, which balances better.
    int local = pl->opt.row_order;
    if (local < 0)
        local = spread && banded_large;
    return make_tasks(pl, n_rows, start, split_cols, shift, n_cu, spread, local != 0);
}

// Kernel 4's groups: block rows taken kGroupRows at a time, greedily by shared
// block columns -- a group starts from the lowest-numbered block row not yet
// placed and adds, one at a time, the unplaced block row sharing the most block
// columns with the group's union so far (ties: the lowest-numbered; a row
// sharing none when no row shares any) -- so that a group's rows need few
// distinct B tiles.  Reads the block-column indices back from the device (a
// synchronous copy).  Fills and uploads the group tables (see kernels.h).
spmm_status_t plan_groups(spmm_plan_s *pl, int64_t nbr, const int32_t *h_ptr, const int32_t *d_idx)
{
    try {
        alloc_probe();
        const int64_t nnzb = h_ptr[nbr];
        std::vector<int32_t> cols((size_t)std::max<int64_t>(1, nnzb));
        if (nnzb > 0) {
            const hipError_t e =
                hipMemcpy(cols.data(), d_idx, sizeof(int32_t) * (size_t)nnzb, hipMemcpyDeviceToHost);
            if (e != hipSuccess)
                return hip_fail(e, "hipMemcpy of the block-column indices");
        }
        const int64_t nbc = ceil_div(pl->k, 64);
        // rows holding each block column (block columns outside [0, k) are kept
        // out of the union: their B rows read as zero and they share nothing)
        std::vector<std::vector<int32_t>> by_col((size_t)std::max<int64_t>(1, nbc));
        for (int64_t r = 0; r < nbr; ++r)
            for (int32_t e = h_ptr[r]; e < h_ptr[r + 1]; ++e)
                if (cols[e] >= 0 && cols[e] < nbc)
                    by_col[cols[e]].push_back((int32_t)r);
        std::vector<char> placed((size_t)nbr, 0);
        std::vector<int32_t> overlap((size_t)nbr, 0), table;
        int64_t next_seed = 0, n_groups = 0;
        while (true) {
            while (next_seed < nbr && placed[next_seed])
                ++next_seed;
            if (next_seed >= nbr)
                break;
            std::vector<int32_t> rows{(int32_t)next_seed};
            placed[next_seed] = 1;
            std::vector<int32_t> uni;
            auto add_cols = [&](int32_t r) {
                for (int32_t e = h_ptr[r]; e < h_ptr[r + 1]; ++e)
                    if (cols[e] >= 0 && cols[e] < nbc &&
                        std::find(uni.begin(), uni.end(), cols[e]) == uni.end())
                        uni.push_back(cols[e]);
            };
            add_cols((int32_t)next_seed);
            while ((int)rows.size() < kGroupRows) {
                // overlap of every unplaced row with the union, through the by-column lists
                std::vector<int32_t> touched;
                for (int32_t c : uni)
                    for (int32_t r : by_col[c])
                        if (!placed[r]) {
                            if (overlap[r]++ == 0)
                                touched.push_back(r);
                        }
                int32_t best = -1;
                for (int32_t r : touched)
                    if (best < 0 || overlap[r] > overlap[best] || (overlap[r] == overlap[best] && r < best))
                        best = r;
                for (int32_t r : touched)
                    overlap[r] = 0;
                if (best < 0) {  // nothing shares a column: the next unplaced row
                    int64_t r = next_seed;
                    while (r < nbr && placed[r])
                        ++r;
                    if (r >= nbr)
                        break;
                    best = (int32_t)r;
                }
                placed[best] = 1;
                rows.push_back(best);
                add_cols(best);
            }
            std::sort(uni.begin(), uni.end());
            std::vector<int32_t> t(kGroupTableInts, 0);
            for (int w = 0; w < kGroupRows; ++w)
                t[w] = w < (int)rows.size() ? rows[w] : -1;
            t[kGroupRows] = (int32_t)uni.size();
            const int maxu = kGroupRows * kGroupMaxBlocks;
            for (size_t u = 0; u < uni.size(); ++u)
                t[kGroupRows + 1 + u] = uni[u];
            for (int w = 0; w < (int)rows.size(); ++w) {
                int q = 0;
                for (int32_t e = h_ptr[rows[w]]; e < h_ptr[rows[w] + 1]; ++e, ++q) {
                    const int32_t c = cols[e];
                    // a block column outside [0, k) contributes nothing: position -1,
                    // the wave skips the block and is no consumer of any item
                    int32_t u = -1;
                    if (c >= 0 && c < nbc) {
                        u = (int32_t)(std::lower_bound(uni.begin(), uni.end(), c) - uni.begin());
                        t[kGroupRows + 1 + maxu + u] += 1;
                    }
                    t[kGroupRows + 1 + 2 * maxu + w * kGroupMaxBlocks + q] = u;
                }
            }
            table.insert(table.end(), t.begin(), t.end());
            ++n_groups;
        }
        pl->n_items = n_groups;
        return upload(table.data(), (int64_t)table.size(), &pl->d_groups);
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
}

// Copies a WCSR plan's values into the tile kernel's A layout (plan-owned,
// b_row * packed entries) on the null stream and waits for the copy.
spmm_status_t pack_values(spmm_plan_s *pl, int64_t nw, const std::vector<int32_t> &pstart, int64_t packed)
{
    if (packed == 0)
        return SPMM_OK;  // no entries: the kernel loads no A
    int32_t *d_pstart = nullptr;
    spmm_status_t s = upload(pstart.data(), nw + 1, &d_pstart);
    if (s != SPMM_OK)
        return s;
    hipError_t e = hipMalloc(&pl->d_apack, (size_t)pl->b_row * (size_t)packed * sizeof(uint16_t));
    if (e != hipSuccess) {
        pl->d_apack = nullptr;
        (void)hipFree(d_pstart);
        return e == hipErrorOutOfMemory ? fail(SPMM_ERR_OUT_OF_MEMORY, "hipMalloc of the packed values")
                                        : hip_fail(e, "hipMalloc of the packed values");
    }
    e = launch_wcsr_pack(pl->A, pl->d_row_ptr, d_pstart, nw, pl->b_row, pl->d_apack, nullptr);
    if (e == hipSuccess)
        e = hipStreamSynchronize(nullptr);
    (void)hipFree(d_pstart);
    if (e != hipSuccess)
        return hip_fail(e, "packing the values");
    pl->A = pl->d_apack;
    return SPMM_OK;
}

// Copies a BCSR plan's 64x64 blocks into the fragment order of the one-wave
// LDS-A kernel (plan-owned, 8 KB per block) on the null stream and waits.
spmm_status_t pack_blocks(spmm_plan_s *pl, int64_t nnzb)
{
    if (nnzb == 0)
        return SPMM_OK;
    if (test_fail_alloc())
        return fail(SPMM_ERR_OUT_OF_MEMORY, "device allocation of the packed blocks refused "
                    "(SPMM_TEST_FAIL_ALLOC)");
    hipError_t e = hipMalloc(&pl->d_apack, (size_t)nnzb * 4096 * sizeof(uint16_t));
    if (e != hipSuccess) {
        pl->d_apack = nullptr;
        return e == hipErrorOutOfMemory ? fail(SPMM_ERR_OUT_OF_MEMORY, "hipMalloc of the packed blocks")
                                        : hip_fail(e, "hipMalloc of the packed blocks");
    }
    e = launch_bcsr64_pack(pl->A, nnzb, pl->d_apack, nullptr);
    if (e == hipSuccess)
        e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess)
        return hip_fail(e, "packing the blocks");
    pl->A = pl->d_apack;
    return SPMM_OK;
}

spmm_plan_s *new_plan(int fmt, int64_t m, int64_t k, int64_t N, int32_t b_row, int32_t b_col,
                      spmm_dtype_t ab, spmm_dtype_t ct, const void *d_vals, const int32_t *d_idx,
                      int dev)
{
    spmm_plan_s *pl = new (std::nothrow) spmm_plan_s();
    if (!pl)
        return nullptr;
    pl->fmt = fmt;
    pl->m = m; pl->k = k; pl->N = N;
    pl->b_row = b_row; pl->b_col = b_col;
    pl->ab = ab; pl->ct = ct;
    pl->A = reinterpret_cast<const uint16_t *>(d_vals);
    pl->col_idx = d_idx;
    pl->device = dev;
    return pl;
}

}  // namespace
}  // namespace wspmm

extern "C" void spmm_plan_options_default(spmm_plan_options_t *opt)
{
    if (!opt)
        return;
    opt->kernel = -1;
    opt->cols_per_lane = 0;
    opt->waves_n = 0;
    opt->waves_k = 0;
    opt->distribution = -1;
    opt->row_order = -1;
    opt->order = -1;
    opt->ranges_per_xcd = 0;
    opt->col_major = 0;
}

extern "C" spmm_status_t spmm_bcsr_plan(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                        int32_t b_row, int32_t b_col,
                                        const int32_t *h_block_row_ptr,
                                        const int32_t *d_block_col_idx, const void *d_blocks,
                                        spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                        size_t *workspace_bytes)
{
    return spmm_bcsr_plan_ex(plan, m, k, N, b_row, b_col, h_block_row_ptr, d_block_col_idx,
                             d_blocks, ab_dtype, c_dtype, nullptr, workspace_bytes);
}

extern "C" spmm_status_t spmm_bcsr_plan_ex(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                           int32_t b_row, int32_t b_col,
                                           const int32_t *h_block_row_ptr,
                                           const int32_t *d_block_col_idx, const void *d_blocks,
                                           spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                           const spmm_plan_options_t *options,
                                           size_t *workspace_bytes)
{
    spmm_status_t s = check_common(plan, m, k, N, b_row, b_col, h_block_row_ptr, d_block_col_idx,
                                   d_blocks, ab_dtype, c_dtype, workspace_bytes, true);
    if (s != SPMM_OK)
        return s;
    *plan = nullptr;
    spmm_plan_options_t opt;
    spmm_plan_options_default(&opt);
    if (options)
        opt = *options;
    if ((s = check_options(opt, true)) != SPMM_OK)
        return s;
    const int64_t nbr = ceil_div(m, b_row);
    const int64_t nnzb = h_block_row_ptr[nbr];
    if (nnzb * b_col >= (int64_t(1) << 31))
        return fail(SPMM_ERR_UNSUPPORTED, "nnz_blocks * b_col must be below 2^31");
    int dev = 0, n_cu = 0;
    int64_t lds_cu = 0, l2 = 0;
    if ((s = current_device(&dev, &n_cu, &lds_cu, &l2)) != SPMM_OK)
        return s;
    spmm_plan_s *pl = new_plan(0, m, k, N, b_row, b_col, ab_dtype, c_dtype, d_blocks,
                               d_block_col_idx, dev);
    if (!pl)
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    pl->opt = opt;
    pl->stored_entries = nnzb * b_row * b_col;
    if ((s = upload(h_block_row_ptr, nbr + 1, &pl->d_row_ptr)) != SPMM_OK) {
        free_plan(pl);
        return s;
    }
    // 64x64 blocks and wide N: kernels that share each A block through LDS and
    // walk whole block rows.
    int max_blocks = 0;
    for (int64_t w = 0; w < nbr; ++w)
        max_blocks = std::max(max_blocks, h_block_row_ptr[w + 1] - h_block_row_ptr[w]);
    const bool b64 = b_row == 64 && b_col == 64;
    pl->max_blocks = max_blocks;
    // Kernel 2 keeps a block row's A in LDS: two resident work-groups per CU
    // are what make each XCD's work-groups sweep the same B tiles together, so
    // it needs every block row to fit twice per CU.
    const int64_t tiles512 = ceil_div(N, 512);
    // kernel 1: 128-column tiles per wave, 2 or 4 waves (N >= 256), or one wave
    // per work-group below N = 256: pinned at any N, and the plan's own choice
    // from N = 128 (16-bit, row-major).  Measured on the P*V workload (65536^2,
    // N = 128, interleaved rounds): 30.9-34.9 us cold and 30.0-30.4 us warm
    // against 34.9-38.6 / 33.2-33.8 us for the generic kernel's best shape (with
    // 9-block-wide lines 180.4 against 193.2 us cold).
    const bool lds_narrow = opt.kernel == -1 && opt.waves_n <= 1 && N >= 128 && !opt.col_major &&
                            ab_dtype != SPMM_FP8_E4M3;
    const bool lds_ok = b64 && (N >= 256 || (opt.kernel == 1 && opt.waves_n <= 1) || lds_narrow);
    // kernel 2 runs 8 columns per lane (512-column tiles), or 4 with col_major
    // or when the options ask for them (256-column tiles, 16-bit inputs)
    const int sweep_v = opt.col_major || opt.cols_per_lane == 4 ? 4 : 8;
    // column-major: 4 waves (256-column tiles, two work-groups per CU) or, as an
    // option, 8 waves (512-column tiles, one work-group per CU)
    const int sweep_nw = opt.col_major && opt.waves_n == 8 ? 8 : 4;
    const bool sweep_fits = b64 && max_blocks <= kSweepMaxBlocks && tiles512 >= 8 &&
                            sweep_blocks_per_cu(ab_dtype, std::max(1, max_blocks), opt.col_major != 0,
                                                sweep_v, sweep_nw) >= (sweep_nw == 8 ? 1 : 2);
    const bool sweep_auto = sweep_fits && tiles512 >= 16;
    // Kernel 3 holds a block row's A in the registers of two waves: at most
    // kPairMaxBlocks blocks per block row, 16-bit inputs, row-major operands,
    // two resident work-groups per CU.
    const bool pair_fits = b64 && max_blocks <= kPairMaxBlocks && N >= 1024 && !opt.col_major &&
                           (ab_dtype == SPMM_FP16 || ab_dtype == SPMM_BF16) &&
                           pair_blocks_per_cu(ab_dtype) >= 2;
    // Kernel 4 groups block rows that share B tiles: at most kGroupMaxBlocks
    // blocks per block row, 16-bit inputs, row-major operands.
    const bool group_fits = b64 && max_blocks <= kGroupMaxBlocks && N >= 1024 && !opt.col_major &&
                            (ab_dtype == SPMM_FP16 || ab_dtype == SPMM_BF16) &&
                            group_blocks_per_cu(ab_dtype) >= 1;
    if (ab_dtype == SPMM_FP8_E4M3 &&
        (!sweep_fits || opt.col_major || (opt.kernel != -1 && opt.kernel != 2))) {
        free_plan(pl);
        return fail(SPMM_ERR_UNSUPPORTED,
                    "FP8_E4M3 runs on the sweep kernel: b_row = b_col = 64, N >= 4096, at most %d "
                    "blocks per block row, row-major B and C", kSweepMaxBlocks);
    }
    if (opt.col_major && (!lds_ok || m % 8 || k % 8 || opt.kernel == 0)) {
        free_plan(pl);
        return fail(SPMM_ERR_UNSUPPORTED,
                    "column-major B and C need b_row = b_col = 64, N >= 256, m and k multiples "
                    "of 8 and kernel 1 or 2");
    }
    pl->kernel = opt.kernel >= 0 ? opt.kernel
                 : sweep_auto || ab_dtype == SPMM_FP8_E4M3 ? 2 : lds_ok ? 1 : 0;
    if ((pl->kernel == 1 && !lds_ok) || (pl->kernel == 2 && !sweep_fits) ||
        (pl->kernel == 3 && !pair_fits) || (pl->kernel == 4 && !group_fits)) {
        free_plan(pl);
        return fail(SPMM_ERR_UNSUPPORTED,
                    "kernel %d cannot run this problem (b_row %d, b_col %d, N %lld, %d blocks in "
                    "the longest block row)",
                    opt.kernel, b_row, b_col, (long long)N, max_blocks);
    }
    if (pl->kernel == 4) {
        if (opt.cols_per_lane != 0 && opt.cols_per_lane != 4) {
            free_plan(pl);
            return fail(SPMM_ERR_UNSUPPORTED, "kernel 4 runs 4 columns per lane");
        }
        if ((s = plan_groups(pl, nbr, h_block_row_ptr, d_block_col_idx)) != SPMM_OK) {
            free_plan(pl);
            return s;
        }
        pl->V = 4;
        pl->waves_n = 1;
        pl->waves_k = 1;
        pl->tile_cols = 64;
        pl->n_col_tiles = ceil_div(N, 64);
        pl->workspace = 0;
        pl->order = 0;
        // ranges of sixteen 64-column strips by default (a block row's A is
        // loaded once per range)
        const int64_t h = opt.ranges_per_xcd > 0
                              ? opt.ranges_per_xcd
                              : std::max<int64_t>(1, std::min<int64_t>(64, pl->n_col_tiles / 128));
        pl->n_ranges = 8 * h;
        pl->range_tiles = ceil_div(pl->n_col_tiles, pl->n_ranges);
    } else if (pl->kernel == 3) {
        if (opt.cols_per_lane != 0 && opt.cols_per_lane != 8) {
            free_plan(pl);
            return fail(SPMM_ERR_UNSUPPORTED, "kernel 3 runs 8 columns per lane");
        }
        pl->n_items = nbr;
        pl->V = 8;
        pl->waves_n = 1;
        pl->waves_k = 2;
        pl->tile_cols = 128;
        pl->n_col_tiles = ceil_div(N, 128);
        pl->workspace = 0;
        pl->order = 0;
        // ranges of eight 128-column strips by default (a block row's A is
        // loaded once per range)
        const int64_t h = opt.ranges_per_xcd > 0
                              ? opt.ranges_per_xcd
                              : std::max<int64_t>(1, std::min<int64_t>(64, pl->n_col_tiles / 64));
        pl->n_ranges = 8 * h;
        pl->range_tiles = ceil_div(pl->n_col_tiles, pl->n_ranges);
    } else if (pl->kernel == 2) {
        // column-major: 4 columns per lane (a whole block of B^T per ring stage)
        if (opt.cols_per_lane != 0 && opt.cols_per_lane != sweep_v) {
            free_plan(pl);
            return fail(SPMM_ERR_UNSUPPORTED, "kernel 2 runs 8 or 4 columns per lane (4 with "
                                              "col_major, 8 with FP8_E4M3)");
        }
        if (ab_dtype == SPMM_FP8_E4M3 && sweep_v != 8) {
            free_plan(pl);
            return fail(SPMM_ERR_UNSUPPORTED, "kernel 2 runs FP8_E4M3 with 8 columns per lane");
        }
        pl->n_items = nbr;
        pl->V = sweep_v;
        pl->waves_n = sweep_nw;
        pl->waves_k = 1;
        pl->tile_cols = 16 * sweep_v * sweep_nw;
        pl->n_col_tiles = ceil_div(N, pl->tile_cols);
        pl->workspace = 0;
        pl->order = 0;
        // Range length.  Longer ranges amortise the A load over more tiles but
        // let the work-groups of an XCD drift apart, so that fewer of them share
        // each B tile in L2; one-tile ranges keep every resident work-group of
        // an XCD on one B slice and re-read A (from L2 and the memory-side
        // cache) once per tile, which pays when A is short and B is wide.
        // Measured on the gate_proj shape (row-major, 6 ranges-per-XCD settings
        // timed interleaved, medians, one box; 1 / 3 / 6 / 8 blocks per block
        // row, N = 8K to 64K, i.e. 16 to 128 tiles):
        //  - about four tiles per range (N / 16384 ranges per XCD) is best or
        //    within 3 % at 1 and 8 blocks, and at 3 and 6 blocks up to 64 and
        //    32 tiles (e.g. 6 blocks, N = 32768: 606 us against 643 us with two
        //    tiles and 656 us with one);
        //  - at 7-8 blocks, past 64 tiles, two ranges per XCD stay best (N =
        //    65536: 1515 us against 1752 us with four tiles, 1598 with one);
        //  - one-tile ranges win at 3-6 blocks from 96 tiles on (6 blocks, N =
        //    65536: 1300 us against 1525 with four tiles; 3 blocks: 885 against
        //    1077) and at 3 blocks from 48 tiles on (N = 32768: 445 against 467).
        // Column-major plans (256-column tiles) count the rule in 512-column
        // units, so that a range spans the columns a row-major range would: on
        // gate_proj two 256-column tiles per range ran 1398-1440 us cold against
        // 1533-1573 us for one (and 1436-1441 us for four).
        const double mean_blocks = (double)h_block_row_ptr[nbr] / (double)std::max<int64_t>(1, nbr);
        const int64_t tiles = opt.col_major ? ceil_div(N, (int64_t)512) : pl->n_col_tiles;
        int64_t h;
        if (opt.ranges_per_xcd > 0) {
            h = opt.ranges_per_xcd;
        } else {
            const bool one_tile = mean_blocks >= 2.5 && ((mean_blocks <= 6.5 && tiles >= 96) ||
                                                         (mean_blocks <= 3.5 && tiles >= 48));
            h = one_tile ? std::min<int64_t>(64, ceil_div(tiles, 8))
                         : std::max<int64_t>(1, std::min<int64_t>(mean_blocks > 6.5 ? 2 : 64, tiles / 32));
        }
        pl->n_ranges = 8 * h;
        pl->range_tiles = ceil_div(pl->n_col_tiles, pl->n_ranges);
    } else if (pl->kernel == 1) {
        if (opt.waves_n > 1 && N < 256) {
            free_plan(pl);
            return fail(SPMM_ERR_UNSUPPORTED, "kernel 1 below N = 256 runs with waves_n = 1 only");
        }
        // 1024-column tiles (8 waves sharing each A block) at wide row-major N
        // and long block rows: measured on down_proj (N = 65536, 30 blocks per
        // block row) 1616-1619 against 1661-1665 us with 512-column tiles (half
        // the A loads and barriers per column); on the gate_proj shape at 80 %
        // block sparsity (11 blocks per block row) 2388-2398 against 2361-2363 us
        // Column-major: 4 columns per lane (a whole block of B^T lines per
        // stage), 8 waves from N = 8192, so that a tile is 512 columns wide.
        const double mean_blocks = (double)h_block_row_ptr[nbr] / (double)std::max<int64_t>(1, nbr);
        const int nw = opt.waves_n > 0 ? opt.waves_n
                       : N < 256 ? 1
                       : opt.col_major ? (N >= 8192 ? 8 : 4)
                       : (N >= 8192 && mean_blocks >= 16.0) ? 8 : 4;
        pl->n_items = nbr;
        pl->V = opt.col_major ? 4 : 8;
        pl->waves_n = nw;
        pl->waves_k = 1;
        pl->tile_cols = 16 * pl->V * nw;
        pl->n_col_tiles = ceil_div(N, pl->tile_cols);
        pl->workspace = 0;
        // one-wave work-groups below N = 256 in launch order (P*V: 30.2-30.4
        // against 37.9 us warm, 30.9-33.9 against 43.6-44.5 us cold, with
        // contiguous ranges per XCD)
        pl->order = opt.order >= 0 ? opt.order : N < 256 ? 1 : 0;
        if (nw == 1 && !opt.col_major && (s = pack_blocks(pl, h_block_row_ptr[nbr])) != SPMM_OK) {
            free_plan(pl);
            return s;
        }
    } else {
        const auto start = [&](int64_t w) { return (int64_t)h_block_row_ptr[w] * b_col; };
        int shift = 0;
        while ((1 << shift) < b_col)
            ++shift;
        if ((s = plan_tasks(pl, nbr, start, 0, std::max(32, (int)b_col), shift, n_cu, lds_cu, l2, h_block_row_ptr)) != SPMM_OK) {
            free_plan(pl);
            return s;
        }
    }
    if (pl->n_items * (pl->kernel >= 2 ? pl->n_ranges : pl->n_col_tiles) > 0x7fffffff) {
        free_plan(pl);
        return fail(SPMM_ERR_UNSUPPORTED, "too many work-groups");
    }
    *workspace_bytes = pl->workspace;
    *plan = pl;
    return ok();
}

extern "C" spmm_status_t spmm_wcsr_plan(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                        int32_t b_row, int32_t b_col,
                                        const int32_t *h_window_row_ptr,
                                        const int32_t *d_window_col_idx, const void *d_values,
                                        spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                        int64_t split_cols, size_t *workspace_bytes)
{
    return spmm_wcsr_plan_ex(plan, m, k, N, b_row, b_col, h_window_row_ptr, d_window_col_idx,
                             d_values, ab_dtype, c_dtype, split_cols, nullptr, workspace_bytes);
}

extern "C" spmm_status_t spmm_wcsr_plan_ex(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                           int32_t b_row, int32_t b_col,
                                           const int32_t *h_window_row_ptr,
                                           const int32_t *d_window_col_idx, const void *d_values,
                                           spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                           int64_t split_cols, const spmm_plan_options_t *options,
                                           size_t *workspace_bytes)
{
    spmm_status_t s = check_common(plan, m, k, N, b_row, b_col, h_window_row_ptr,
                                   d_window_col_idx, d_values, ab_dtype, c_dtype, workspace_bytes,
                                   false);
    if (s != SPMM_OK)
        return s;
    *plan = nullptr;
    spmm_plan_options_t opt;
    spmm_plan_options_default(&opt);
    if (options)
        opt = *options;
    if ((s = check_options(opt, false)) != SPMM_OK)
        return s;
    if (split_cols < 0 || split_cols % 32 != 0 || split_cols > kMaxSplit)
        return fail(SPMM_ERR_INVALID_ARGUMENT,
                    "split_cols must be 0 or a positive multiple of 32 up to %lld",
                    (long long)kMaxSplit);
    int dev = 0, n_cu = 0;
    int64_t lds_cu = 0, l2 = 0;
    if ((s = current_device(&dev, &n_cu, &lds_cu, &l2)) != SPMM_OK)
        return s;
    const int64_t nw = ceil_div(m, b_row);
    const int64_t P = h_window_row_ptr[nw];
    const auto start = [&](int64_t w) { return (int64_t)h_window_row_ptr[w]; };
    spmm_plan_s *pl = new_plan(1, m, k, N, b_row, b_col, ab_dtype, c_dtype, d_values,
                               d_window_col_idx, dev);
    if (!pl)
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    pl->opt = opt;
    pl->stored_entries = P * b_row;
    int64_t widest = 0;
    for (int64_t w = 0; w < nw; ++w)
        widest = std::max<int64_t>(widest, (int64_t)h_window_row_ptr[w + 1] - h_window_row_ptr[w]);
    if ((uint64_t)widest * (uint64_t)b_row * 2u >= kMaxBBytes) {
        free_plan(pl);
        return fail(SPMM_ERR_UNSUPPORTED, "a window tile (b_row * width * 2 bytes) must be below 4 GiB");
    }
    // The values in the tile kernel's A layout: window w at entry b_row *
    // pstart[w], its width rounded up to whole 32-column steps.
    std::vector<int32_t> pstart;
    try {
        pstart.resize((size_t)nw + 1);
    } catch (const std::bad_alloc &) {
        free_plan(pl);
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    int64_t packed = 0;
    for (int64_t w = 0; w < nw; ++w) {
        pstart[w] = (int32_t)packed;
        packed += ceil_div((int64_t)h_window_row_ptr[w + 1] - h_window_row_ptr[w], 32) * 32;
        if (packed > 0x7fffffff) {
            free_plan(pl);
            return fail(SPMM_ERR_UNSUPPORTED, "more than 2^31 - 1 packed columns after rounding windows to 32");
        }
    }
    pstart[nw] = (int32_t)packed;
    pl->h_pstart = &pstart;
    if ((s = upload(h_window_row_ptr, nw + 1, &pl->d_row_ptr)) != SPMM_OK ||
        (s = plan_tasks(pl, nw, start, split_cols, 32, 0, n_cu, lds_cu, l2, h_window_row_ptr)) != SPMM_OK ||
        (s = pack_values(pl, nw, pstart, packed)) != SPMM_OK) {
        free_plan(pl);
        return s;
    }
    pl->h_pstart = nullptr;
    if (pl->n_items * (pl->kernel >= 2 ? pl->n_ranges : pl->n_col_tiles) > 0x7fffffff) {
        free_plan(pl);
        return fail(SPMM_ERR_UNSUPPORTED, "too many work-groups");
    }
    *workspace_bytes = pl->workspace;
    *plan = pl;
    return ok();
}

extern "C" spmm_status_t spmm_bcsr_run(spmm_plan_t plan, const void *d_B, int64_t ldb, void *d_C,
                                       int64_t ldc, void *d_workspace, void *stream)
{
    return run_plan(plan, 0, d_B, ldb, d_C, ldc, d_workspace, stream);
}

extern "C" spmm_status_t spmm_wcsr_run(spmm_plan_t plan, const void *d_B, int64_t ldb, void *d_C,
                                       int64_t ldc, void *d_workspace, void *stream)
{
    return run_plan(plan, 1, d_B, ldb, d_C, ldc, d_workspace, stream);
}

// ---------------------------------------------------------------------------
// Tuned plans.  The plan's own rules pick one configuration per problem from
// its shape; the paper instead measures throughput against the tile width and
// keeps the best one (Section IV-C, Fig. 7).  These entry points make that
// measurement on the caller's operands: every configuration the caller's
// options leave open is planned and timed on the caller's stream, and the
// fastest plan is kept.
namespace wspmm {
namespace {

// A candidate keeps every field the caller pinned; a candidate that pins a
// field to another value than the caller's is dropped.
bool merge_pinned(const spmm_plan_options_t &base, spmm_plan_options_t &o)
{
    auto field = [](int32_t b, int32_t &c, int32_t automatic) {
        if (b == automatic)
            return true;
        if (c == automatic)
            c = b;
        return c == b;
    };
    return field(base.kernel, o.kernel, -1) && field(base.cols_per_lane, o.cols_per_lane, 0) &&
           field(base.waves_n, o.waves_n, 0) && field(base.waves_k, o.waves_k, 0) &&
           field(base.distribution, o.distribution, -1) && field(base.row_order, o.row_order, -1) &&
           field(base.order, o.order, -1) && field(base.ranges_per_xcd, o.ranges_per_xcd, 0) &&
           field(base.col_major, o.col_major, 0);
}

// The configurations to time after the automatic one: the 64 x 64 block
// kernels' variants (BCSR with 64 x 64 blocks), then the generic kernel's tile
// shapes (columns per lane x waves across the tile x waves along the packed
// columns, with both ways of handing out tasks).  Configurations a kernel
// cannot run are refused by the plan and skipped.
std::vector<spmm_plan_options_t> tune_candidates(const spmm_plan_options_t &base, bool bcsr,
                                                 int32_t b_row, int32_t b_col)
{
    std::vector<spmm_plan_options_t> out;
    auto add = [&](spmm_plan_options_t o) {
        if (!merge_pinned(base, o))
            return;
        for (const auto &x : out)
            if (std::memcmp(&x, &o, sizeof(o)) == 0)
                return;
        out.push_back(o);
    };
    spmm_plan_options_t o;
    if (bcsr && b_row == 64 && b_col == 64) {
        for (int wn : {1, 2, 4, 8})
            for (int ord : {0, 1}) {
                spmm_plan_options_default(&o);
                o.kernel = 1; o.waves_n = wn; o.order = ord;
                add(o);
            }
        for (int cpl : {8, 4})
            for (int h : {1, 2, 4, 8, 16}) {
                spmm_plan_options_default(&o);
                o.kernel = 2; o.cols_per_lane = cpl; o.ranges_per_xcd = h;
                add(o);
            }
        if (base.col_major == 1)   // the sweep kernel's 8-wave column-major tiles
            for (int h : {1, 2, 4, 8, 16}) {
                spmm_plan_options_default(&o);
                o.kernel = 2; o.waves_n = 8; o.ranges_per_xcd = h;
                add(o);
            }
        for (int kern : {3, 4})
            for (int h : {1, 2, 4, 8, 16, 32}) {
                spmm_plan_options_default(&o);
                o.kernel = kern; o.ranges_per_xcd = h;
                add(o);
            }
    }
    static const int kWaves[6][2] = {{1, 1}, {1, 2}, {1, 4}, {2, 1}, {2, 2}, {4, 1}};
    for (int V : {2, 4, 8}) {
        if (V == 8 && b_row >= 32)
            continue;
        for (const auto &w : kWaves)
            for (int dist : {0, 1}) {
                spmm_plan_options_default(&o);
                o.kernel = 0; o.cols_per_lane = V; o.waves_n = w[0]; o.waves_k = w[1];
                o.distribution = dist;
                add(o);
            }
    }
    return out;
}

// Device memory and events of one tuning call, released on every return path.
struct TuneState {
    void *ws = nullptr;
    size_t ws_cap = 0;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    ~TuneState()
    {
        if (ws) (void)hipFree(ws);
        if (e0) (void)hipEventDestroy(e0);
        if (e1) (void)hipEventDestroy(e1);
    }
    // a workspace of at least n bytes (grows, never shrinks)
    spmm_status_t reserve(size_t n)
    {
        if (n <= ws_cap)
            return SPMM_OK;
        if (ws) (void)hipFree(ws);
        ws = nullptr;
        ws_cap = 0;
        if (test_fail_alloc() || hipMalloc(&ws, n) != hipSuccess) {
            ws = nullptr;
            return fail(SPMM_ERR_OUT_OF_MEMORY, "tuning workspace of %zu bytes", n);
        }
        ws_cap = n;
        return SPMM_OK;
    }
};

// Mean time (us) of one run of `pl`: two untimed runs, then `reps` runs
// between two events on the stream.
spmm_status_t time_runs(spmm_plan_t pl, const void *B, int64_t ldb, void *C, int64_t ldc,
                        TuneState &ts, void *stream, int reps, double *us)
{
    spmm_status_t s = ts.reserve(pl->workspace);
    if (s != SPMM_OK)
        return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int i = 0; i < 2; ++i)
        if ((s = run_plan(pl, pl->fmt, B, ldb, C, ldc, ts.ws, stream)) != SPMM_OK)
            return s;
    hipError_t e = hipEventRecord(ts.e0, st);
    for (int i = 0; e == hipSuccess && i < reps; ++i)
        if ((s = run_plan(pl, pl->fmt, B, ldb, C, ldc, ts.ws, stream)) != SPMM_OK)
            return s;
    if (e == hipSuccess)
        e = hipEventRecord(ts.e1, st);
    if (e == hipSuccess)
        e = hipEventSynchronize(ts.e1);
    float ms = 0.f;
    if (e == hipSuccess)
        e = hipEventElapsedTime(&ms, ts.e0, ts.e1);
    if (e != hipSuccess)
        return hip_fail(e, "timing a candidate plan");
    *us = (double)ms * 1e3 / reps;
    return SPMM_OK;
}

using PlanMaker = std::function<spmm_status_t(const spmm_plan_options_t &, int64_t, spmm_plan_t *)>;

// A candidate replaces the incumbent only when it is this much faster, so that
// timing noise does not trade the automatic plan for an equal one.
constexpr double kTuneMargin = 0.02;
// Candidates kept after the first timing, and rounds of the final comparison.
constexpr int kTuneFinalists = 4;
constexpr int kTuneRounds = 3;

struct Timed {
    spmm_plan_t plan;
    spmm_plan_options_t opt;
    double us;
};

// One selection stage: every candidate (options, split size) is planned and
// timed once; the fastest kTuneFinalists are then timed again kTuneRounds
// times, interleaved with the incumbent, and the one with the lowest median
// replaces the incumbent if it is kTuneMargin faster.  Candidates no kernel
// can run (UNSUPPORTED or INVALID_ARGUMENT from the plan) and candidates whose
// plan or workspace cannot be allocated are skipped; other errors end the
// stage.
spmm_status_t select_plan(const PlanMaker &make,
                          const std::vector<std::pair<spmm_plan_options_t, int64_t>> &cands,
                          const void *B, int64_t ldb, void *C, int64_t ldc, TuneState &ts,
                          void *stream, int n, Timed &inc, int *timed)
{
    std::vector<Timed> top;  // sorted by time, at most kTuneFinalists
    auto release = [&]() {
        for (auto &t : top)
            free_plan(t.plan);
        top.clear();
    };
    for (const auto &cand : cands) {
        spmm_plan_t c = nullptr;
        spmm_status_t r = make(cand.first, cand.second, &c);
        // (OUT_OF_MEMORY: its tables or value copy do not fit beside the
        // plans already held -- not a candidate either)
        if (r == SPMM_ERR_UNSUPPORTED || r == SPMM_ERR_INVALID_ARGUMENT || r == SPMM_ERR_OUT_OF_MEMORY)
            continue;
        if (r != SPMM_OK) {
            release();
            return r;
        }
        double us = 0.0;
        r = time_runs(c, B, ldb, C, ldc, ts, stream, n, &us);
        if (r != SPMM_OK) {
            free_plan(c);
            if (r == SPMM_ERR_OUT_OF_MEMORY)  // its workspace does not fit: not a candidate
                continue;
            release();
            return r;
        }
        ++*timed;
        top.push_back({c, cand.first, us});
        std::sort(top.begin(), top.end(), [](const Timed &a, const Timed &b) { return a.us < b.us; });
        if ((int)top.size() > kTuneFinalists) {
            free_plan(top.back().plan);
            top.pop_back();
        }
    }
    if (top.empty())
        return SPMM_OK;
    // final rounds: incumbent and finalists in turn, median of the rounds
    std::vector<std::vector<double>> t(top.size() + 1);
    for (int round = 0; round < kTuneRounds; ++round)
        for (size_t i = 0; i <= top.size(); ++i) {
            double us = 0.0;
            spmm_status_t r = time_runs(i == 0 ? inc.plan : top[i - 1].plan, B, ldb, C, ldc, ts,
                                        stream, n, &us);
            if (r != SPMM_OK) {
                release();
                return r;
            }
            t[i].push_back(us);
        }
    auto median = [](std::vector<double> v) {
        std::sort(v.begin(), v.end());
        return v[v.size() / 2];
    };
    inc.us = median(t[0]);
    size_t best = 0;
    double best_us = inc.us * (1.0 - kTuneMargin);
    for (size_t i = 1; i <= top.size(); ++i) {
        const double us = median(t[i]);
        if (us < best_us) {
            best = i;
            best_us = us;
        }
    }
    if (best > 0) {
        free_plan(inc.plan);
        inc = top[best - 1];
        inc.us = best_us;
        top[best - 1].plan = nullptr;
    }
    for (auto &x : top)
        if (x.plan)
            free_plan(x.plan);
    top.clear();
    return SPMM_OK;
}

spmm_status_t tune_plan(int fmt, int32_t b_row, int32_t b_col, const PlanMaker &make,
                        const spmm_plan_options_t *options, int64_t split_cols, const void *B,
                        int64_t ldb, void *C, int64_t ldc, void *stream, int32_t reps,
                        spmm_plan_options_t *chosen, spmm_plan_t *plan, size_t *workspace_bytes)
{
    if (reps < 0 || reps > 10000)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "reps must be in [0, 10000]");
    spmm_plan_options_t base;
    spmm_plan_options_default(&base);
    if (options)
        base = *options;
    Timed inc{nullptr, base, 0.0};
    spmm_status_t s = make(base, split_cols, &inc.plan);
    if (s != SPMM_OK)
        return s;
    // the operands must suit the plan before anything is launched (a stand-in
    // workspace address: the tuner brings its own)
    if ((s = check_run(inc.plan, B, ldb, C, ldc, inc.plan->workspace ? (void *)16 : nullptr)) !=
        SPMM_OK) {
        free_plan(inc.plan);
        return s;
    }
    auto done = [&](spmm_status_t st, int timed) {
        if (st != SPMM_OK) {
            free_plan(inc.plan);
            return st;
        }
        inc.plan->n_tuned = timed;
        *plan = inc.plan;
        *workspace_bytes = inc.plan->workspace;
        if (chosen)
            *chosen = inc.opt;
        return ok();
    };
    if (inc.plan->m == 0 || inc.plan->N == 0 || inc.plan->n_items == 0)
        return done(SPMM_OK, 0);
    TuneState ts;
    hipError_t e = hipEventCreate(&ts.e0);
    if (e == hipSuccess)
        e = hipEventCreate(&ts.e1);
    if (e != hipSuccess)
        return done(hip_fail(e, "event creation"), 0);
    // reps: enough runs for about 4 ms of timed work (at least 5), from a
    // 3-run probe: candidates of one kernel differ by a few per cent
    if ((s = time_runs(inc.plan, B, ldb, C, ldc, ts, stream, 3, &inc.us)) != SPMM_OK)
        return done(s, 0);
    const int n = reps > 0 ? reps
                           : (int)std::min(100.0, std::max(5.0, 4000.0 / std::max(inc.us, 1.0)));
    int timed = 1;
    std::vector<std::pair<spmm_plan_options_t, int64_t>> cands;
    for (const auto &o : tune_candidates(base, fmt == 0, b_row, b_col))
        cands.emplace_back(o, split_cols);
    if ((s = select_plan(make, cands, B, ldb, C, ldc, ts, stream, n, inc, &timed)) != SPMM_OK)
        return done(s, timed);
    // WCSR with an automatic split size: the sub-task size as a second stage,
    // with the configuration the first stage kept
    if (fmt == 1 && split_cols == 0 && inc.plan->kernel == 0) {
        cands.clear();
        for (int64_t T : {128, 512, 2048, 8192})
            cands.emplace_back(inc.opt, T);
        if ((s = select_plan(make, cands, B, ldb, C, ldc, ts, stream, n, inc, &timed)) != SPMM_OK)
            return done(s, timed);
    }
    return done(SPMM_OK, timed);
}

}  // namespace
}  // namespace wspmm

extern "C" spmm_status_t spmm_bcsr_plan_tuned(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                              int32_t b_row, int32_t b_col,
                                              const int32_t *h_block_row_ptr,
                                              const int32_t *d_block_col_idx, const void *d_blocks,
                                              spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                              const spmm_plan_options_t *options, const void *d_B,
                                              int64_t ldb, void *d_C, int64_t ldc, void *stream,
                                              int32_t reps, spmm_plan_options_t *chosen,
                                              size_t *workspace_bytes)
{
    if (!plan || !workspace_bytes)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null plan or workspace_bytes pointer");
    *plan = nullptr;
    size_t ws = 0;
    const PlanMaker make = [&](const spmm_plan_options_t &o, int64_t, spmm_plan_t *out) {
        return spmm_bcsr_plan_ex(out, m, k, N, b_row, b_col, h_block_row_ptr, d_block_col_idx,
                                 d_blocks, ab_dtype, c_dtype, &o, &ws);
    };
    return tune_plan(0, b_row, b_col, make, options, 0, d_B, ldb, d_C, ldc, stream, reps, chosen,
                     plan, workspace_bytes);
}

extern "C" spmm_status_t spmm_wcsr_plan_tuned(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                              int32_t b_row, int32_t b_col,
                                              const int32_t *h_window_row_ptr,
                                              const int32_t *d_window_col_idx, const void *d_values,
                                              spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                              int64_t split_cols, const spmm_plan_options_t *options,
                                              const void *d_B, int64_t ldb, void *d_C, int64_t ldc,
                                              void *stream, int32_t reps,
                                              spmm_plan_options_t *chosen, size_t *workspace_bytes)
{
    if (!plan || !workspace_bytes)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null plan or workspace_bytes pointer");
    *plan = nullptr;
    size_t ws = 0;
    const PlanMaker make = [&](const spmm_plan_options_t &o, int64_t T, spmm_plan_t *out) {
        return spmm_wcsr_plan_ex(out, m, k, N, b_row, b_col, h_window_row_ptr, d_window_col_idx,
                                 d_values, ab_dtype, c_dtype, T, &o, &ws);
    };
    return tune_plan(1, b_row, b_col, make, options, split_cols, d_B, ldb, d_C, ldc, stream, reps,
                     chosen, plan, workspace_bytes);
}

// ---------------------------------------------------------------------------
// The run that allocates nothing: the fp32 partial tiles of split windows go
// into this file's static device array instead of a caller-supplied
// workspace.  Each GPU the library runs on holds its own copy of the array
// until the process ends; host code never passes the array's name to a
// kernel (in host code it only stands in for the symbol), but the device
// address looked up once per device.
namespace {
constexpr size_t kScratchBytes = SPMM_NOALLOC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_address[kMaxDevices];               // per device, null until looked up
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
// Device address of `scratch` on device dev (which must be current).
spmm_status_t scratch_address(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SPMM_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_address[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(SPMM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_address[dev] = ptr;
    }
    *out = g_scratch_address[dev];
    return SPMM_OK;
}
}  // namespace

extern "C" spmm_status_t spmm_wcsr_run_noalloc(spmm_plan_t plan, const void *d_B, int64_t ldb,
                                               void *d_C, int64_t ldc, void *stream)
{
    if (!plan)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null plan");
    if (plan->fmt != 1)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "spmm_wcsr_run_noalloc takes a WCSR plan");
    if (plan->workspace > kScratchBytes)
        return fail(SPMM_ERR_UNSUPPORTED,
                    "the plan needs %zu bytes of partial tiles; the static scratch holds %zu "
                    "(use spmm_wcsr_run with a workspace, or a plan with a larger split size)",
                    plan->workspace, kScratchBytes);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "plan was made on device %d, current is %d",
                    plan->device, dev);
    void *ws = nullptr;
    if (plan->workspace > 0 && plan->m > 0 && plan->N > 0) {
        const spmm_status_t s = scratch_address(dev, &ws);
        if (s != SPMM_OK)
            return s;
    }
    return run_plan(plan, 1, d_B, ldb, d_C, ldc, ws, stream);
}

extern "C" spmm_status_t spmm_plan_info(spmm_plan_t pl, spmm_plan_info_t *info)
{
    if (!pl || !info)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null plan or info");
    std::memset(info, 0, sizeof(*info));
    info->format = pl->fmt;
    info->tile_rows = pl->b_row;
    info->tile_cols = (int32_t)pl->tile_cols;
    info->waves_n = pl->waves_n;
    info->waves_k = pl->waves_k;
    info->cols_per_lane = pl->V;
    info->kernel = pl->kernel;
    info->ranges_per_xcd = pl->kernel >= 2 ? (int32_t)(pl->n_ranges / 8) : 0;
    info->col_major = pl->opt.col_major;
    info->split_cols = pl->kernel == 0 ? pl->split_cols : 0;
    info->n_tasks = pl->kernel == 0 ? pl->n_tasks : 0;
    info->n_merges = pl->n_merges;
    info->n_slots = pl->n_slots;
    info->stored_entries = pl->stored_entries;
    info->workspace_bytes = pl->workspace;
    info->tuned = pl->n_tuned;
    return ok();
}

extern "C" spmm_status_t spmm_plan_destroy(spmm_plan_t plan)
{
    free_plan(plan);
    return ok();
}

namespace wspmm {
namespace {
// The empty kernel behind spmm_launch_floor.
__global__ void launch_floor_kernel() {}
}  // namespace
}  // namespace wspmm

extern "C" spmm_status_t spmm_launch_floor(void *stream)
{
    hipLaunchKernelGGL(wspmm::launch_floor_kernel, dim3(1), dim3(64), 0,
                       reinterpret_cast<hipStream_t>(stream));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? ok() : hip_fail(e, "empty kernel launch");
}

extern "C" int64_t spmm_recommended_ld(int64_t N, int32_t elem_bytes)
{
    if (N <= 0 || elem_bytes <= 0)
        return N;
    const int64_t ld = ceil_div(N, 8) * 8;
    if ((ld * elem_bytes) % 4096 != 0)
        return ld;
    // A row pitch that is a multiple of 4 KiB puts the rows of a column slice
    // into the same L2 sets.  From 16 KiB on, the pitch gets half a 4 KiB page
    // more: rows then alternate between the two halves of a page, and the time
    // of a run no longer depends on where in memory B and C sit (with one
    // 128-byte line more, the same run varied up to 2x between allocations).
    // Shorter pitches get the one line (64 elements, 128 for 1-byte data), at
    // a smaller cost in memory.
    if (ld * elem_bytes >= 16384)
        return ld + ceil_div(ceil_div(2048, elem_bytes), 8) * 8;
    return ld + (elem_bytes == 1 ? 128 : 64);
}

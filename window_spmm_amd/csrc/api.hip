// C-ABI entry points: plans and runs for BCSR and WCSR SpMM on gfx950.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <functional>
#include <cstring>
#include <new>
#include <vector>

#include "common.h"
#include "kernels.h"

struct spmm_plan_s {
    int fmt;                    // 0 = BCSR, 1 = WCSR
    int64_t m, k, N;
    int32_t b_row, b_col;
    int ab, ct;
    const uint16_t *A;
    const int32_t *col_idx;
    int32_t *d_row_ptr;         // plan-owned copy of the block / window row pointer
    int32_t *d_tasks;           // WCSR (window, begin, end, slot)
    int32_t *d_merges;          // WCSR (window, first_slot, n_slots)
    int64_t n_items;            // block rows (BCSR) or tasks (WCSR)
    int64_t n_merges, n_slots, split_cols;
    int64_t lds_idx_ints;       // LDS index area of the generic kernel (ints)
    int64_t stored_entries;
    int V, waves_n, waves_k;
    int kernel;                 // 0: generic tile kernel, 1: BCSR 64x64 with LDS-shared A
    int64_t tile_cols, n_col_tiles;
    size_t workspace;
    int device;
};

namespace wspmm {
namespace {

// Buffer resources address at most 2^32 bytes; the kernels use offsets above
// this bound as "read zero".
constexpr uint64_t kMaxBBytes = 0xFFFFFF00ull;

int env_int(const char *name, int dflt)
{
    const char *s = std::getenv(name);
    return (s && *s) ? std::atoi(s) : dflt;
}

spmm_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(SPMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The library only runs on gfx950; find out whether the current device is one.
spmm_status_t current_device(int *dev, int *n_cu)
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
    if (ab != SPMM_FP16 && ab != SPMM_BF16)
        return fail(SPMM_ERR_UNSUPPORTED, "A/B dtype must be FP16 or BF16");
    if (ct != SPMM_FP32 && ct != SPMM_BF16 && ct != SPMM_FP16)
        return fail(SPMM_ERR_UNSUPPORTED, "C dtype must be FP32, BF16 or FP16");
    if (N % 8 != 0)
        return fail(SPMM_ERR_UNSUPPORTED, "N = %lld must be a multiple of 8", (long long)N);
    if (N > (int64_t(1) << 28) || m >= (int64_t(1) << 31) || k >= (int64_t(1) << 31))
        return fail(SPMM_ERR_UNSUPPORTED, "matrix dimension too large");
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
void choose_config(spmm_plan_s *pl, double mean_kprime, int n_cu)
{
    int V = pl->N >= 128 ? 8 : (pl->N >= 64 ? 4 : 2);
    V = env_int("SPMM_FORCE_V", V);
    if (V != 2 && V != 4 && V != 8)
        V = 8;
    const int64_t wave_cols = 16 * V;
    const int64_t col_waves = ceil_div(pl->N, wave_cols);
    int wn = (pl->b_row == 64 && col_waves >= 2) ? 2 : 1;
    wn = std::max(1, std::min(4, env_int("SPMM_FORCE_WAVES_N", wn)));
    const int64_t col_tiles = std::max<int64_t>(1, ceil_div(pl->N, wave_cols * wn));
    // add reduction waves while the grid is small and the items are long
    const int64_t waves = std::max<int64_t>(1, pl->n_items * col_tiles * wn);
    int wk = 1;
    while (wn * wk * 2 <= 4 && waves * wk < int64_t(16) * n_cu && mean_kprime >= 64.0 * wk * 2)
        wk *= 2;
    wk = std::max(1, std::min(4 / wn, env_int("SPMM_FORCE_WAVES_K", wk)));
    pl->V = V;
    pl->waves_n = wn;
    pl->waves_k = wk;
    pl->tile_cols = wave_cols * wn;
    pl->n_col_tiles = pl->N > 0 ? ceil_div(pl->N, pl->tile_cols) : 0;
}

template <typename T>
spmm_status_t upload(const T *h, int64_t n, T **d)
{
    *d = nullptr;
    if (n == 0)
        return SPMM_OK;
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
    if (pl->d_merges) (void)hipFree(pl->d_merges);
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
    if (ldb < pl->N || ldc < pl->N || ldb % 8 || ldc % 8)
        return fail(SPMM_ERR_UNSUPPORTED, "ldb/ldc must be >= N and multiples of 8");
    if ((uint64_t)pl->k * (uint64_t)ldb * 2u >= kMaxBBytes)
        return fail(SPMM_ERR_UNSUPPORTED, "B (k * ldb * 2 bytes) must be smaller than 4 GiB - 256");
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
    p.tasks = reinterpret_cast<const int4 *>(pl->d_tasks);
    p.B = reinterpret_cast<const uint16_t *>(B);
    p.ldb = ldb;
    p.C = C;
    p.ldc = ldc;
    p.partial = reinterpret_cast<float *>(ws);
    p.m = pl->m;
    p.k = pl->k;
    p.N = pl->N;
    p.b_bytes = (uint64_t)pl->k * (uint64_t)ldb * 2u;
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
    p.order = env_int("SPMM_FORCE_ORDER", 0) ? 1 : 0;
    p.lds_idx_ints = (int32_t)pl->lds_idx_ints;
    hipError_t e = pl->kernel == 1 ? launch_bcsr64_lds(pl->ab, p, st)
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

// Sub-task size when the caller leaves it to the plan.  If the longest row tile
// is within 4x the mean width, T covers it (no tile is cut, no merge pass);
// otherwise T is twice the mean, so only the long tail is cut.  T is a multiple
// of `align`, at least 512 and at most kMaxSplit.
constexpr int64_t kMaxSplit = 8192;

int64_t auto_split(int64_t n_rows, const std::function<int64_t(int64_t)> &start, int64_t align)
{
    int64_t total = start(n_rows) - start(0), longest = 0;
    for (int64_t w = 0; w < n_rows; ++w)
        longest = std::max(longest, start(w + 1) - start(w));
    const int64_t mean = n_rows > 0 ? ceil_div(total, n_rows) : 0;
    int64_t T = longest <= 4 * mean ? longest : 2 * mean;
    T = std::max<int64_t>(512, ceil_div(T, align) * align);
    T = std::min<int64_t>(T, kMaxSplit);
    const int64_t forced = env_int("SPMM_FORCE_SPLIT", 0);
    if (forced > 0 && forced % align == 0 && forced <= kMaxSplit)
        T = forced;
    return T;
}

// Splits the row tiles into tasks (row tile w covers packed columns
// [start(w), start(w+1))), uploads task and merge tables, sizes the LDS index
// area (`shift`: log2 of packed columns per index entry) and the workspace.
spmm_status_t make_tasks(spmm_plan_s *pl, int64_t n_rows, const std::function<int64_t(int64_t)> &start,
                         int64_t split_cols, int shift)
{
    try {
        std::vector<int32_t> tasks, merges;
        split_tasks(n_rows, start, split_cols, tasks, merges);
        const int64_t nt = (int64_t)tasks.size() / 4, nm = (int64_t)merges.size() / 3;
        int64_t slots = 0, max_idx = 0;
        for (int64_t i = 0; i < nm; ++i)
            slots += merges[3 * i + 2];
        for (int64_t i = 0; i < nt; ++i)
            max_idx = std::max<int64_t>(max_idx, (int64_t)(tasks[4 * i + 2] - tasks[4 * i + 1]) >> shift);
        pl->n_items = nt;
        pl->n_merges = nm;
        pl->n_slots = slots;
        pl->split_cols = split_cols;
        // the staging copies whole 256-entry runs; index reads start at most 8 before the end
        pl->lds_idx_ints = ceil_div(max_idx, 256) * 256 + 256;
        spmm_status_t s;
        if ((s = upload(tasks.data(), nt * 4, &pl->d_tasks)) != SPMM_OK ||
            (s = upload(merges.data(), nm * 3, &pl->d_merges)) != SPMM_OK)
            return s;
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    if (pl->n_merges > 0 && ceil_div((int64_t)pl->b_row * (pl->N / 8), 256) > 65535)
        return fail(SPMM_ERR_UNSUPPORTED, "N too large for the merge grid");
    pl->workspace = (size_t)pl->n_slots * (size_t)pl->b_row * (size_t)pl->N * sizeof(float);
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

extern "C" spmm_status_t spmm_bcsr_plan(spmm_plan_t *plan, int64_t m, int64_t k, int64_t N,
                                        int32_t b_row, int32_t b_col,
                                        const int32_t *h_block_row_ptr,
                                        const int32_t *d_block_col_idx, const void *d_blocks,
                                        spmm_dtype_t ab_dtype, spmm_dtype_t c_dtype,
                                        size_t *workspace_bytes)
{
    spmm_status_t s = check_common(plan, m, k, N, b_row, b_col, h_block_row_ptr, d_block_col_idx,
                                   d_blocks, ab_dtype, c_dtype, workspace_bytes, true);
    if (s != SPMM_OK)
        return s;
    *plan = nullptr;
    const int64_t nbr = ceil_div(m, b_row);
    const int64_t nnzb = h_block_row_ptr[nbr];
    if (nnzb * b_col >= (int64_t(1) << 31))
        return fail(SPMM_ERR_UNSUPPORTED, "nnz_blocks * b_col must be below 2^31");
    int dev = 0, n_cu = 0;
    if ((s = current_device(&dev, &n_cu)) != SPMM_OK)
        return s;
    spmm_plan_s *pl = new_plan(0, m, k, N, b_row, b_col, ab_dtype, c_dtype, d_blocks,
                               d_block_col_idx, dev);
    if (!pl)
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    pl->stored_entries = nnzb * b_row * b_col;
    if ((s = upload(h_block_row_ptr, nbr + 1, &pl->d_row_ptr)) != SPMM_OK) {
        free_plan(pl);
        return s;
    }
    // 64x64 blocks and at least one full 256-column tile: the kernel that shares
    // each A block through LDS walks whole block rows
    pl->kernel = env_int("SPMM_FORCE_KERNEL", (b_row == 64 && b_col == 64 && N >= 256) ? 1 : 0);
    if (pl->kernel == 1 && b_row == 64 && b_col == 64) {
        const int nw = env_int("SPMM_FORCE_WAVES_N", 4) == 2 ? 2 : 4;
        pl->n_items = nbr;
        pl->V = 8;
        pl->waves_n = nw;
        pl->waves_k = 1;
        pl->tile_cols = 128 * nw;
        pl->n_col_tiles = ceil_div(N, pl->tile_cols);
        pl->workspace = 0;
    } else {
        pl->kernel = 0;
        const int align = std::max(32, (int)b_col);
        const auto start = [&](int64_t w) { return (int64_t)h_block_row_ptr[w] * b_col; };
        const int64_t T = auto_split(nbr, start, align);
        int shift = 0;
        while ((1 << shift) < b_col)
            ++shift;
        if ((s = make_tasks(pl, nbr, start, T, shift)) != SPMM_OK) {
            free_plan(pl);
            return s;
        }
        const double mean_task = pl->n_items > 0 ? (double)(nnzb * b_col) / pl->n_items : 0.0;
        choose_config(pl, mean_task, n_cu);
    }
    if (pl->n_items * pl->n_col_tiles > 0x7fffffff) {
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
    spmm_status_t s = check_common(plan, m, k, N, b_row, b_col, h_window_row_ptr,
                                   d_window_col_idx, d_values, ab_dtype, c_dtype, workspace_bytes,
                                   false);
    if (s != SPMM_OK)
        return s;
    *plan = nullptr;
    if (split_cols < 0 || split_cols % 32 != 0 || split_cols > kMaxSplit)
        return fail(SPMM_ERR_INVALID_ARGUMENT,
                    "split_cols must be 0 or a positive multiple of 32 up to %lld",
                    (long long)kMaxSplit);
    int dev = 0, n_cu = 0;
    if ((s = current_device(&dev, &n_cu)) != SPMM_OK)
        return s;
    const int64_t nw = ceil_div(m, b_row);
    const int64_t P = h_window_row_ptr[nw];
    const auto start = [&](int64_t w) { return (int64_t)h_window_row_ptr[w]; };
    if (split_cols == 0)
        split_cols = auto_split(nw, start, 32);
    spmm_plan_s *pl = new_plan(1, m, k, N, b_row, b_col, ab_dtype, c_dtype, d_values,
                               d_window_col_idx, dev);
    if (!pl)
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    pl->stored_entries = P * b_row;
    if ((s = upload(h_window_row_ptr, nw + 1, &pl->d_row_ptr)) != SPMM_OK ||
        (s = make_tasks(pl, nw, start, split_cols, 0)) != SPMM_OK) {
        free_plan(pl);
        return s;
    }
    const double mean_task = pl->n_items > 0 ? (double)P / (double)pl->n_items : 0.0;
    choose_config(pl, mean_task, n_cu);
    if (pl->n_items * pl->n_col_tiles > 0x7fffffff) {
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
    info->split_cols = pl->kernel == 0 ? pl->split_cols : 0;
    info->n_tasks = pl->kernel == 0 ? pl->n_items : 0;
    info->n_merges = pl->n_merges;
    info->n_slots = pl->n_slots;
    info->stored_entries = pl->stored_entries;
    info->workspace_bytes = pl->workspace;
    return ok();
}

extern "C" spmm_status_t spmm_plan_destroy(spmm_plan_t plan)
{
    free_plan(plan);
    return ok();
}

extern "C" int64_t spmm_recommended_ld(int64_t N, int32_t elem_bytes)
{
    if (N <= 0 || elem_bytes <= 0)
        return N;
    const int64_t ld = ceil_div(N, 8) * 8;
    // Row pitches that are a multiple of 4 KiB put the rows of a column slice into
    // the same L2 sets; 64 extra elements (an odd number of 128-byte lines for
    // 16-bit data) spread them.
    return (ld * elem_bytes) % 4096 == 0 ? ld + 64 : ld;
}

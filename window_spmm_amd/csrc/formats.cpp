// Host-side construction of the two sparse formats of the AsyncSparse paper
// (Section II-C, Fig. 2) from CSR, and the window-splitting task list of
// Section III-C.  Integer work only: values are 16-bit codes copied verbatim.
#include <algorithm>
#include <cstring>
#include <functional>
#include <new>
#include <vector>

#include "common.h"

namespace wspmm {

spmm_status_t validate_csr(int64_t m, int64_t k, const int32_t *row_ptr, const int32_t *col_idx)
{
    if (m < 0 || k < 0)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "negative matrix size (m=%lld, k=%lld)",
                    (long long)m, (long long)k);
    if (!row_ptr)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "row_ptr is null");
    if (row_ptr[0] != 0)
        return fail(SPMM_ERR_BAD_FORMAT, "row_ptr[0] = %d, expected 0", row_ptr[0]);
    for (int64_t i = 0; i < m; ++i)
        if (row_ptr[i + 1] < row_ptr[i])
            return fail(SPMM_ERR_BAD_FORMAT, "row_ptr decreases at row %lld", (long long)i);
    if (row_ptr[m] > 0 && !col_idx)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "col_idx is null");
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t) {
            int32_t c = col_idx[t];
            if (c < 0 || c >= k)
                return fail(SPMM_ERR_BAD_FORMAT, "column %d out of range [0, %lld) in row %lld", c,
                            (long long)k, (long long)i);
            if (t > row_ptr[i] && c <= col_idx[t - 1])
                return fail(SPMM_ERR_BAD_FORMAT, "columns of row %lld not strictly increasing",
                            (long long)i);
        }
    }
    return SPMM_OK;
}

namespace {

spmm_status_t check_block_dims(int32_t b_row, int32_t b_col)
{
    if (b_row < 1 || b_row > 1024 || b_col < 1 || b_col > 1024)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "block/window size %d x %d outside [1, 1024]", b_row,
                    b_col);
    return SPMM_OK;
}

// Distinct block columns touched by rows [r0, r1), increasing.  `mark` has one
// slot per block column and holds the stamp of the last block row that used it.
void block_columns(const int32_t *row_ptr, const int32_t *col_idx, int64_t r0, int64_t r1,
                   int32_t b_col, int64_t stamp, std::vector<int64_t> &mark,
                   std::vector<int32_t> &out)
{
    out.clear();
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t) {
            int32_t J = col_idx[t] / b_col;
            if (mark[J] != stamp) {
                mark[J] = stamp;
                out.push_back(J);
            }
        }
    std::sort(out.begin(), out.end());
}

// Distinct columns of rows [r0, r1), increasing (the window's column union).
void window_union(const int32_t *row_ptr, const int32_t *col_idx, int64_t r0, int64_t r1,
                  int64_t stamp, std::vector<int64_t> &mark, std::vector<int32_t> &out)
{
    out.clear();
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t) {
            int32_t c = col_idx[t];
            if (mark[c] != stamp) {
                mark[c] = stamp;
                out.push_back(c);
            }
        }
    std::sort(out.begin(), out.end());
}

}  // namespace
}  // namespace wspmm

using namespace wspmm;

extern "C" spmm_status_t spmm_csr_to_bcsr_count(int64_t m, int64_t k, const int32_t *row_ptr,
                                                const int32_t *col_idx, int32_t b_row,
                                                int32_t b_col, int64_t *nnz_blocks)
{
    if (!nnz_blocks)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "nnz_blocks is null");
    spmm_status_t s = check_block_dims(b_row, b_col);
    if (s == SPMM_OK)
        s = validate_csr(m, k, row_ptr, col_idx);
    if (s != SPMM_OK)
        return s;
    try {
        alloc_probe();
        const int64_t nbr = ceil_div(m, b_row), nbc = ceil_div(k, b_col);
        std::vector<int64_t> mark(nbc > 0 ? nbc : 1, -1);
        std::vector<int32_t> cols;
        int64_t total = 0;
        for (int64_t I = 0; I < nbr; ++I) {
            block_columns(row_ptr, col_idx, I * b_row, std::min<int64_t>(m, (I + 1) * b_row),
                          b_col, I, mark, cols);
            total += (int64_t)cols.size();
        }
        if (total >= (int64_t(1) << 31))
            return fail(SPMM_ERR_UNSUPPORTED, "nnz_blocks = %lld does not fit int32",
                        (long long)total);
        *nnz_blocks = total;
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

namespace {

// The BCSR fill for codes of type T (16-bit or 8-bit values, copied bit-exactly).
template <typename T>
spmm_status_t bcsr_fill(int64_t m, int64_t k, const int32_t *row_ptr, const int32_t *col_idx,
                        const T *values, int32_t b_row, int32_t b_col, int32_t *block_row_ptr,
                        int32_t *block_col_idx, T *blocks)
{
    int64_t nnzb = 0;
    spmm_status_t s = spmm_csr_to_bcsr_count(m, k, row_ptr, col_idx, b_row, b_col, &nnzb);
    if (s != SPMM_OK)
        return s;
    if (!block_row_ptr || (nnzb > 0 && (!block_col_idx || !blocks)) || (row_ptr[m] > 0 && !values))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null output or values pointer");
    try {
        alloc_probe();
        const int64_t nbr = ceil_div(m, b_row), nbc = ceil_div(k, b_col);
        const int64_t bsz = (int64_t)b_row * b_col;
        std::vector<int64_t> mark(nbc > 0 ? nbc : 1, -1);
        std::vector<int32_t> slot(nbc > 0 ? nbc : 1, 0);
        std::vector<int32_t> cols;
        int64_t next = 0;
        block_row_ptr[0] = 0;
        for (int64_t I = 0; I < nbr; ++I) {
            const int64_t r0 = I * b_row, r1 = std::min<int64_t>(m, (I + 1) * b_row);
            block_columns(row_ptr, col_idx, r0, r1, b_col, I, mark, cols);
            for (size_t q = 0; q < cols.size(); ++q) {
                block_col_idx[next + (int64_t)q] = cols[q];
                slot[cols[q]] = (int32_t)q;
            }
            if (cols.empty()) {
                block_row_ptr[I + 1] = (int32_t)next;
                continue;
            }
            T *base = blocks + next * bsz;
            std::memset(base, 0, sizeof(T) * bsz * cols.size());
            for (int64_t i = r0; i < r1; ++i)
                for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t) {
                    const int32_t c = col_idx[t];
                    base[(int64_t)slot[c / b_col] * bsz + (i - r0) * b_col + c % b_col] = values[t];
                }
            next += (int64_t)cols.size();
            block_row_ptr[I + 1] = (int32_t)next;
        }
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

}  // namespace

extern "C" spmm_status_t spmm_csr_to_bcsr(int64_t m, int64_t k, const int32_t *row_ptr,
                                          const int32_t *col_idx, const uint16_t *values,
                                          int32_t b_row, int32_t b_col, int32_t *block_row_ptr,
                                          int32_t *block_col_idx, uint16_t *blocks)
{
    return bcsr_fill<uint16_t>(m, k, row_ptr, col_idx, values, b_row, b_col, block_row_ptr,
                               block_col_idx, blocks);
}

extern "C" spmm_status_t spmm_csr_to_bcsr8(int64_t m, int64_t k, const int32_t *row_ptr,
                                           const int32_t *col_idx, const uint8_t *values,
                                           int32_t b_row, int32_t b_col, int32_t *block_row_ptr,
                                           int32_t *block_col_idx, uint8_t *blocks)
{
    return bcsr_fill<uint8_t>(m, k, row_ptr, col_idx, values, b_row, b_col, block_row_ptr,
                              block_col_idx, blocks);
}

extern "C" spmm_status_t spmm_csr_to_wcsr_count(int64_t m, int64_t k, const int32_t *row_ptr,
                                                const int32_t *col_idx, int32_t b_row,
                                                int32_t b_col, int64_t *padded_cols)
{
    if (!padded_cols)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "padded_cols is null");
    spmm_status_t s = check_block_dims(b_row, b_col);
    if (s == SPMM_OK)
        s = validate_csr(m, k, row_ptr, col_idx);
    if (s != SPMM_OK)
        return s;
    try {
        alloc_probe();
        const int64_t nw = ceil_div(m, b_row);
        std::vector<int64_t> mark(k > 0 ? k : 1, -1);
        std::vector<int32_t> cols;
        int64_t P = 0;
        for (int64_t w = 0; w < nw; ++w) {
            window_union(row_ptr, col_idx, w * b_row, std::min<int64_t>(m, (w + 1) * b_row), w,
                         mark, cols);
            P += ceil_div((int64_t)cols.size(), b_col) * b_col;
        }
        if (P >= (int64_t(1) << 31))
            return fail(SPMM_ERR_UNSUPPORTED, "padded column count %lld does not fit int32",
                        (long long)P);
        *padded_cols = P;
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

extern "C" spmm_status_t spmm_csr_to_wcsr(int64_t m, int64_t k, const int32_t *row_ptr,
                                          const int32_t *col_idx, const uint16_t *values,
                                          int32_t b_row, int32_t b_col, int32_t *window_row_ptr,
                                          int32_t *window_col_idx, uint16_t *values_out)
{
    int64_t P = 0;
    spmm_status_t s = spmm_csr_to_wcsr_count(m, k, row_ptr, col_idx, b_row, b_col, &P);
    if (s != SPMM_OK)
        return s;
    if (!window_row_ptr || (P > 0 && (!window_col_idx || !values_out)) ||
        (row_ptr[m] > 0 && !values))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null output or values pointer");
    try {
        alloc_probe();
        const int64_t nw = ceil_div(m, b_row);
        std::vector<int64_t> mark(k > 0 ? k : 1, -1);
        std::vector<int32_t> pos(k > 0 ? k : 1, 0);
        std::vector<int32_t> cols;
        int64_t p0 = 0;
        window_row_ptr[0] = 0;
        for (int64_t w = 0; w < nw; ++w) {
            const int64_t r0 = w * b_row, r1 = std::min<int64_t>(m, (w + 1) * b_row);
            window_union(row_ptr, col_idx, r0, r1, w, mark, cols);
            const int64_t n = (int64_t)cols.size();
            const int64_t W = ceil_div(n, b_col) * b_col;
            for (int64_t q = 0; q < n; ++q) {
                window_col_idx[p0 + q] = cols[q];
                pos[cols[q]] = (int32_t)q;
            }
            for (int64_t q = n; q < W; ++q)
                window_col_idx[p0 + q] = -1;
            if (W == 0) {
                window_row_ptr[w + 1] = (int32_t)p0;
                continue;
            }
            uint16_t *tile = values_out + (int64_t)b_row * p0;
            std::memset(tile, 0, sizeof(uint16_t) * (size_t)(b_row * W));
            for (int64_t i = r0; i < r1; ++i)
                for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t)
                    tile[(i - r0) * W + pos[col_idx[t]]] = values[t];
            p0 += W;
            window_row_ptr[w + 1] = (int32_t)p0;
        }
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

namespace {

spmm_status_t check_split_args(int64_t n_windows, const int32_t *wptr, int64_t split_cols)
{
    if (n_windows < 0 || !wptr)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "bad window count or null window_row_ptr");
    if (split_cols <= 0 || split_cols % 32 != 0 || split_cols >= (int64_t(1) << 31))
        return fail(SPMM_ERR_INVALID_ARGUMENT,
                    "split_cols = %lld must be a positive multiple of 32", (long long)split_cols);
    if (wptr[0] != 0)
        return fail(SPMM_ERR_BAD_FORMAT, "window_row_ptr[0] = %d, expected 0", wptr[0]);
    for (int64_t w = 0; w < n_windows; ++w)
        if (wptr[w + 1] < wptr[w])
            return fail(SPMM_ERR_BAD_FORMAT, "window_row_ptr decreases at window %lld",
                        (long long)w);
    return SPMM_OK;
}

}  // namespace

namespace wspmm {

void split_tasks(int64_t n_rows, const std::function<int64_t(int64_t)> &start, int64_t split_cols,
                 std::vector<int32_t> &tasks, std::vector<int32_t> &merges)
{
    tasks.clear();
    merges.clear();
    int64_t slot = 0;
    for (int64_t w = 0; w < n_rows; ++w) {
        const int64_t p0 = start(w), p1 = start(w + 1);
        if (p1 - p0 <= split_cols) {
            tasks.insert(tasks.end(), {(int32_t)w, (int32_t)p0, (int32_t)p1, -1});
            continue;
        }
        const int64_t parts = ceil_div(p1 - p0, split_cols);
        merges.insert(merges.end(), {(int32_t)w, (int32_t)slot, (int32_t)parts});
        for (int64_t q = 0; q < parts; ++q)
            tasks.insert(tasks.end(), {(int32_t)w, (int32_t)(p0 + q * split_cols),
                                       (int32_t)std::min(p1, p0 + (q + 1) * split_cols),
                                       (int32_t)(slot + q)});
        slot += parts;
    }
}

}  // namespace wspmm

extern "C" spmm_status_t spmm_wcsr_split_count(int64_t n_windows, const int32_t *wptr,
                                               int64_t split_cols, int64_t *n_tasks,
                                               int64_t *n_merges)
{
    if (!n_tasks || !n_merges)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null count pointer");
    spmm_status_t s = check_split_args(n_windows, wptr, split_cols);
    if (s != SPMM_OK)
        return s;
    int64_t nt = 0, nm = 0;
    for (int64_t w = 0; w < n_windows; ++w) {
        const int64_t W = (int64_t)wptr[w + 1] - wptr[w];
        if (W <= split_cols) {
            nt += 1;
        } else {
            nt += ceil_div(W, split_cols);
            nm += 1;
        }
    }
    *n_tasks = nt;
    *n_merges = nm;
    return ok();
}

extern "C" spmm_status_t spmm_wcsr_split(int64_t n_windows, const int32_t *wptr,
                                         int64_t split_cols, int32_t *tasks, int32_t *merges)
{
    int64_t nt = 0, nm = 0;
    spmm_status_t s = spmm_wcsr_split_count(n_windows, wptr, split_cols, &nt, &nm);
    if (s != SPMM_OK)
        return s;
    if ((nt > 0 && !tasks) || (nm > 0 && !merges))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null tasks or merges pointer");
    try {
        alloc_probe();
        std::vector<int32_t> t, m;
        split_tasks(n_windows, [wptr](int64_t w) { return (int64_t)wptr[w]; }, split_cols, t, m);
        std::copy(t.begin(), t.end(), tasks);
        std::copy(m.begin(), m.end(), merges);
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

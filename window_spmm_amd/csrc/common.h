// Internal helpers shared by the host-side sources of the library.
#pragma once

#include <functional>
#include <new>
#include <vector>

#include "window_spmm.h"

namespace wspmm {

// Records a thread-local message for spmm_last_error() and returns `s`.
spmm_status_t fail(spmm_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread-local message and returns SPMM_OK.
spmm_status_t ok();

// Test hook for the out-of-memory paths: when the environment variable
// SPMM_TEST_FAIL_ALLOC is set to anything but "" or "0", every allocation
// the library guards fails (host allocations throw std::bad_alloc from here,
// device allocations report failure), so that the OUT_OF_MEMORY handling
// can be exercised without exhausting memory.  A no-op otherwise.
bool test_fail_alloc();
inline void alloc_probe()
{
    if (test_fail_alloc())
        throw std::bad_alloc();
}

// Checks a CSR pattern: row_ptr[0] = 0, non-decreasing, columns in [0, k) and
// strictly increasing inside every row.
spmm_status_t validate_csr(int64_t m, int64_t k, const int32_t *row_ptr, const int32_t *col_idx);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The window-splitting rule (see spmm_wcsr_split) over any row pointer:
// start(w) is the first packed column of row tile w, start(n_rows) the end.
// Appends (tile, begin, end, slot) to tasks and (tile, first_slot, n_slots) to merges.
void split_tasks(int64_t n_rows, const std::function<int64_t(int64_t)> &start, int64_t split_cols,
                 std::vector<int32_t> &tasks, std::vector<int32_t> &merges);

}  // namespace wspmm

// Host-side reordering: reverse Cuthill-McKee order of a square CSR pattern and
// the symmetric permutation P A P^T (AsyncSparse paper, Section IV-A: every
// evaluation matrix is reordered with reverse Cuthill-McKee before the formats
// are built, to bring nonzeros closer to the diagonal; the method is Cuthill and
// McKee's breadth-first numbering, reversed).
#include <algorithm>
#include <cstdint>
#include <new>
#include <utility>
#include <vector>

#include "common.h"

namespace wspmm {
namespace {

// Adjacency of G = pattern(A) + pattern(A)^T without self loops, each list
// sorted and free of repeats (CSR form: off[n + 1], nbr[off[n]]).
struct Graph {
    std::vector<int64_t> off;
    std::vector<int32_t> nbr;
    int64_t deg(int32_t v) const { return off[v + 1] - off[v]; }
};

void symmetrize(int64_t n, const int32_t *row_ptr, const int32_t *col_idx, Graph &g)
{
    std::vector<int64_t> cnt(n + 1, 0);
    for (int64_t i = 0; i < n; ++i)
        for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const int32_t j = col_idx[e];
            if (j == i)
                continue;
            ++cnt[i + 1];
            ++cnt[j + 1];
        }
    for (int64_t i = 0; i < n; ++i)
        cnt[i + 1] += cnt[i];
    std::vector<int32_t> all(cnt[n]);
    std::vector<int64_t> pos(cnt.begin(), cnt.end() - 1);
    for (int64_t i = 0; i < n; ++i)
        for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const int32_t j = col_idx[e];
            if (j == i)
                continue;
            all[pos[i]++] = j;
            all[pos[j]++] = (int32_t)i;
        }
    g.off.assign(n + 1, 0);
    g.nbr.clear();
    g.nbr.reserve(all.size());
    for (int64_t i = 0; i < n; ++i) {
        auto b = all.begin() + cnt[i], e = all.begin() + cnt[i + 1];
        std::sort(b, e);
        auto last = std::unique(b, e);
        g.nbr.insert(g.nbr.end(), b, last);
        g.off[i + 1] = (int64_t)g.nbr.size();
    }
}

// Breadth-first level structure rooted at r inside r's component: fills
// `order` with the component's vertices in breadth-first order, `level` with
// each one's distance from r, and returns the height (the last level's index).
// `mark`/`stamp` avoid clearing per search.
int64_t levels(const Graph &g, int32_t r, std::vector<int32_t> &order, std::vector<int64_t> &level,
               std::vector<int64_t> &mark, int64_t stamp)
{
    order.clear();
    order.push_back(r);
    mark[r] = stamp;
    level[r] = 0;
    int64_t h = 0;
    for (size_t q = 0; q < order.size(); ++q) {
        const int32_t v = order[q];
        for (int64_t e = g.off[v]; e < g.off[v + 1]; ++e) {
            const int32_t w = g.nbr[e];
            if (mark[w] != stamp) {
                mark[w] = stamp;
                level[w] = level[v] + 1;
                h = level[w];
                order.push_back(w);
            }
        }
    }
    return h;
}

}  // namespace
}  // namespace wspmm

using namespace wspmm;

extern "C" spmm_status_t spmm_rcm_order(int64_t n, const int32_t *row_ptr, const int32_t *col_idx,
                                        int32_t *perm)
{
    if (n < 0)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (n == 0)
        return ok();
    if (!row_ptr || !perm || (row_ptr[n] > 0 && !col_idx))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null pointer");
    if (n >= (int64_t(1) << 31))
        return fail(SPMM_ERR_UNSUPPORTED, "n must be below 2^31");
    spmm_status_t s = validate_csr(n, n, row_ptr, col_idx);
    if (s != SPMM_OK)
        return s;
    try {
        alloc_probe();
        Graph g;
        symmetrize(n, row_ptr, col_idx, g);
        std::vector<char> placed(n, 0);
        std::vector<int64_t> mark(n, -1), level(n, 0);
        std::vector<int32_t> comp, tmp, kids;
        int64_t stamp = 0, out = 0;
        // vertices by (degree, index): the first one not yet placed starts the
        // next component
        std::vector<int32_t> by_deg(n);
        for (int64_t i = 0; i < n; ++i)
            by_deg[i] = (int32_t)i;
        std::stable_sort(by_deg.begin(), by_deg.end(),
                         [&](int32_t a, int32_t b) { return g.deg(a) < g.deg(b); });
        auto less_deg = [&](int32_t a, int32_t b) {
            return g.deg(a) != g.deg(b) ? g.deg(a) < g.deg(b) : a < b;
        };
        size_t next = 0;
        while (out < n) {
            while (placed[by_deg[next]])
                ++next;
            int32_t r = by_deg[next];
            // pseudo-peripheral vertex (George and Liu): move to the least-degree
            // vertex of the last level while that lengthens the level structure
            int64_t h = levels(g, r, comp, level, mark, stamp++);
            for (;;) {
                int32_t x = -1;
                for (int32_t v : comp)
                    if (level[v] == h && (x < 0 || less_deg(v, x)))
                        x = v;
                const int64_t hx = levels(g, x, tmp, level, mark, stamp++);
                if (hx <= h)
                    break;
                r = x;
                h = hx;
                comp.swap(tmp);
            }
            // Cuthill-McKee: breadth first from r, each vertex's unplaced
            // neighbours appended by increasing (degree, index)
            const int64_t first = out;
            perm[out++] = r;
            placed[r] = 1;
            for (int64_t q = first; q < out; ++q) {
                const int32_t v = perm[q];
                kids.clear();
                for (int64_t e = g.off[v]; e < g.off[v + 1]; ++e)
                    if (!placed[g.nbr[e]])
                        kids.push_back(g.nbr[e]);
                std::sort(kids.begin(), kids.end(), less_deg);
                for (int32_t w : kids) {
                    placed[w] = 1;
                    perm[out++] = w;
                }
            }
        }
        std::reverse(perm, perm + n);
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

extern "C" spmm_status_t spmm_csr_permute(int64_t n, const int32_t *row_ptr, const int32_t *col_idx,
                                          const uint16_t *values, const int32_t *perm,
                                          int32_t *out_row_ptr, int32_t *out_col_idx,
                                          uint16_t *out_values)
{
    if (n < 0)
        return fail(SPMM_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (!row_ptr || (n > 0 && (!perm || !out_row_ptr)) || (row_ptr[n] > 0 && !col_idx))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null pointer");
    if (n >= (int64_t(1) << 31))
        return fail(SPMM_ERR_UNSUPPORTED, "n must be below 2^31");
    spmm_status_t s = validate_csr(n, n, row_ptr, col_idx);
    if (s != SPMM_OK)
        return s;
    if (n == 0) {
        if (out_row_ptr)
            out_row_ptr[0] = 0;
        return ok();
    }
    const int64_t nnz = row_ptr[n];
    if (nnz > 0 && (!values || !out_col_idx || !out_values))
        return fail(SPMM_ERR_INVALID_ARGUMENT, "null pointer");
    try {
        alloc_probe();
        std::vector<int32_t> inv(n, -1);
        for (int64_t i = 0; i < n; ++i) {
            const int32_t p = perm[i];
            if (p < 0 || p >= n || inv[p] >= 0)
                return fail(SPMM_ERR_INVALID_ARGUMENT, "perm is not a permutation of 0..n-1");
            inv[p] = (int32_t)i;
        }
        out_row_ptr[0] = 0;
        std::vector<std::pair<int32_t, uint16_t>> row;
        for (int64_t i = 0; i < n; ++i) {
            const int32_t src = perm[i];
            row.clear();
            for (int32_t e = row_ptr[src]; e < row_ptr[src + 1]; ++e)
                row.emplace_back(inv[col_idx[e]], values[e]);
            std::sort(row.begin(), row.end(),
                      [](const std::pair<int32_t, uint16_t> &a, const std::pair<int32_t, uint16_t> &b) {
                          return a.first < b.first;
                      });
            int32_t at = out_row_ptr[i];
            for (const auto &x : row) {
                out_col_idx[at] = x.first;
                out_values[at] = x.second;
                ++at;
            }
            out_row_ptr[i + 1] = at;
        }
    } catch (const std::bad_alloc &) {
        return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    return ok();
}

// Driver for the sanitizer build of the library's host code (format builders,
// window split, reordering and status handling).  Built with
// -fsanitize=address,undefined together with the library's host sources and
// run by tests/test_sanitizers.py: random CSR patterns of many shapes go
// through every builder (count, then fill), the encodings are decoded back and
// compared with the input, and malformed inputs must be refused with an error
// code.  Any out-of-bounds access, leak, overflow or other undefined behaviour
// aborts the run.  Prints "ok" at the end.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "window_spmm.h"

static int g_fail = 0;
#define EXPECT(c)                                                              \
    do {                                                                       \
        if (!(c)) {                                                            \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++g_fail;                                                          \
        }                                                                      \
    } while (0)

struct Csr {
    int64_t m, k;
    std::vector<int32_t> ptr, idx;
    std::vector<uint16_t> val;
};

static Csr random_csr(std::mt19937_64 &g, int64_t m, int64_t k, double dens)
{
    Csr a{m, k, {0}, {}, {}};
    std::uniform_real_distribution<double> u(0.0, 1.0);
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < k; ++j)
            if (u(g) < dens) {
                a.idx.push_back((int32_t)j);
                a.val.push_back((uint16_t)(1 + g() % 0x7BFF));  // a nonzero code
            }
        a.ptr.push_back((int32_t)a.idx.size());
    }
    return a;
}

static void check_bcsr(const Csr &a, int br, int bc)
{
    int64_t nb = -1;
    EXPECT(spmm_csr_to_bcsr_count(a.m, a.k, a.ptr.data(), a.idx.data(), br, bc, &nb) == SPMM_OK);
    const int64_t nbr = (a.m + br - 1) / br;
    std::vector<int32_t> bptr(nbr + 1), bidx(nb > 0 ? nb : 1);
    std::vector<uint16_t> blk(nb > 0 ? nb * br * bc : 1);
    std::vector<uint8_t> blk8(nb > 0 ? nb * br * bc : 1);
    std::vector<uint8_t> val8(a.val.size() + 1);
    for (size_t e = 0; e < a.val.size(); ++e)
        val8[e] = (uint8_t)(1 + a.val[e] % 0x7E);
    EXPECT(spmm_csr_to_bcsr(a.m, a.k, a.ptr.data(), a.idx.data(), a.val.data(), br, bc, bptr.data(),
                            bidx.data(), blk.data()) == SPMM_OK);
    EXPECT(spmm_csr_to_bcsr8(a.m, a.k, a.ptr.data(), a.idx.data(), val8.data(), br, bc, bptr.data(),
                             bidx.data(), blk8.data()) == SPMM_OK);
    // decode: every CSR entry sits in its block, and the count of stored
    // nonzero codes equals nnz
    int64_t nonzero = 0;
    for (int64_t q = 0; q < nb * br * bc; ++q)
        nonzero += blk[q] != 0;
    EXPECT(nonzero == (int64_t)a.val.size());
    for (int64_t i = 0; i < a.m; ++i)
        for (int32_t e = a.ptr[i]; e < a.ptr[i + 1]; ++e) {
            const int64_t I = i / br, J = a.idx[e] / bc;
            int64_t q = -1;
            for (int32_t t = bptr[I]; t < bptr[I + 1]; ++t)
                if (bidx[t] == J)
                    q = t;
            EXPECT(q >= 0);
            if (q >= 0) {
                const int64_t off = (q * br + i % br) * bc + a.idx[e] % bc;
                EXPECT(blk[off] == a.val[e]);
                EXPECT(blk8[off] == val8[e]);
            }
        }
}

static void check_wcsr(const Csr &a, int br, int bc)
{
    int64_t P = -1;
    EXPECT(spmm_csr_to_wcsr_count(a.m, a.k, a.ptr.data(), a.idx.data(), br, bc, &P) == SPMM_OK);
    const int64_t nw = (a.m + br - 1) / br;
    std::vector<int32_t> wptr(nw + 1), widx(P > 0 ? P : 1);
    std::vector<uint16_t> wv(P > 0 ? P * br : 1);
    EXPECT(spmm_csr_to_wcsr(a.m, a.k, a.ptr.data(), a.idx.data(), a.val.data(), br, bc, wptr.data(),
                            widx.data(), wv.data()) == SPMM_OK);
    int64_t nonzero = 0;
    for (int64_t q = 0; q < P * br; ++q)
        nonzero += wv[q] != 0;
    EXPECT(nonzero == (int64_t)a.val.size());
    for (int64_t i = 0; i < a.m; ++i)
        for (int32_t e = a.ptr[i]; e < a.ptr[i + 1]; ++e) {
            const int64_t w = i / br, W = wptr[w + 1] - wptr[w];
            int64_t p = -1;
            for (int32_t t = wptr[w]; t < wptr[w + 1]; ++t)
                if (widx[t] == a.idx[e])
                    p = t - wptr[w];
            EXPECT(p >= 0);
            if (p >= 0)
                EXPECT(wv[br * (int64_t)wptr[w] + (i % br) * W + p] == a.val[e]);
        }
    for (int64_t T : {32, 64, 96, 512}) {
        int64_t nt = -1, nm = -1;
        EXPECT(spmm_wcsr_split_count(nw, wptr.data(), T, &nt, &nm) == SPMM_OK);
        std::vector<int32_t> tasks(nt * 4 + 1), merges(nm * 3 + 1);
        EXPECT(spmm_wcsr_split(nw, wptr.data(), T, tasks.data(), merges.data()) == SPMM_OK);
        int64_t covered = 0;
        for (int64_t t = 0; t < nt; ++t) {
            EXPECT(tasks[4 * t + 2] - tasks[4 * t + 1] <= T);
            covered += tasks[4 * t + 2] - tasks[4 * t + 1];
        }
        EXPECT(covered == P);
    }
}

static void check_reorder(const Csr &a)
{
    std::vector<int32_t> perm(a.m + 1);
    EXPECT(spmm_rcm_order(a.m, a.ptr.data(), a.idx.data(), perm.data()) == SPMM_OK);
    std::vector<char> seen(a.m + 1, 0);
    for (int64_t i = 0; i < a.m; ++i) {
        EXPECT(perm[i] >= 0 && perm[i] < a.m);
        if (perm[i] >= 0 && perm[i] < a.m)
            seen[perm[i]] = 1;
    }
    for (int64_t i = 0; i < a.m; ++i)
        EXPECT(seen[i]);
    std::vector<int32_t> optr(a.m + 1), oidx(a.idx.size() + 1);
    std::vector<uint16_t> oval(a.val.size() + 1);
    EXPECT(spmm_csr_permute(a.m, a.ptr.data(), a.idx.data(), a.val.data(), perm.data(), optr.data(),
                            oidx.data(), oval.data()) == SPMM_OK);
    EXPECT(optr[a.m] == (int32_t)a.idx.size());
}

static void check_errors()
{
    // unsorted / duplicate / out-of-range columns, bad row pointer, bad sizes, nulls
    const int32_t ptr[] = {0, 2, 3}, unsorted[] = {3, 1, 2}, dup[] = {1, 1, 2}, oor[] = {0, 9, 2};
    const int32_t back[] = {0, 3, 2};
    int64_t n = 0;
    EXPECT(spmm_csr_to_bcsr_count(2, 8, ptr, unsorted, 2, 2, &n) == SPMM_ERR_BAD_FORMAT);
    EXPECT(spmm_csr_to_wcsr_count(2, 8, ptr, dup, 2, 2, &n) == SPMM_ERR_BAD_FORMAT);
    EXPECT(spmm_csr_to_wcsr_count(2, 8, ptr, oor, 2, 2, &n) == SPMM_ERR_BAD_FORMAT);
    EXPECT(spmm_csr_to_bcsr_count(2, 8, back, unsorted, 2, 2, &n) == SPMM_ERR_BAD_FORMAT);
    EXPECT(spmm_csr_to_bcsr_count(-1, 8, ptr, unsorted, 2, 2, &n) == SPMM_ERR_INVALID_ARGUMENT);
    EXPECT(spmm_csr_to_bcsr_count(2, 8, nullptr, unsorted, 2, 2, &n) == SPMM_ERR_INVALID_ARGUMENT);
    EXPECT(spmm_csr_to_wcsr_count(2, 8, ptr, dup, 0, 2, &n) == SPMM_ERR_INVALID_ARGUMENT);
    int64_t nt = 0, nm = 0;
    EXPECT(spmm_wcsr_split_count(2, back, 32, &nt, &nm) == SPMM_ERR_BAD_FORMAT);
    EXPECT(spmm_wcsr_split_count(1, ptr, 40, &nt, &nm) != SPMM_OK);
    int32_t perm[2];
    const int32_t sq_ptr[] = {0, 1, 2}, sq_idx[] = {1, 0};
    const int32_t bad_perm[] = {0, 0};
    uint16_t v[2] = {1, 2}, ov[2];
    int32_t optr[3], oidx[2];
    EXPECT(spmm_rcm_order(2, sq_ptr, sq_idx, perm) == SPMM_OK);
    EXPECT(spmm_csr_permute(2, sq_ptr, sq_idx, v, bad_perm, optr, oidx, ov) == SPMM_ERR_INVALID_ARGUMENT);
    EXPECT(spmm_last_error()[0] != '\0');
    EXPECT(spmm_status_string((spmm_status_t)77)[0] != '\0');
}

int main()
{
    std::mt19937_64 g(20261203);
    const int shapes[][2] = {{0, 0}, {1, 1}, {1, 37}, {37, 1}, {63, 64}, {64, 64}, {65, 130}, {200, 90}};
    const int blocks[][2] = {{1, 1}, {16, 8}, {16, 16}, {32, 8}, {64, 64}, {3, 5}};
    for (int rep = 0; rep < 3; ++rep)
        for (auto &s : shapes)
            for (double d : {0.0, 0.02, 0.3, 1.0}) {
                const Csr a = random_csr(g, s[0], s[1], d);
                for (auto &b : blocks) {
                    check_bcsr(a, b[0], b[1]);
                    check_wcsr(a, b[0], b[1]);
                }
                if (a.m == a.k) {
                    // the reordering takes a square pattern
                    check_reorder(a);
                }
            }
    for (int sq : {2, 33, 128}) {
        const Csr a = random_csr(g, sq, sq, 0.05);
        check_reorder(a);
    }
    check_errors();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}

// gfx950 BCSR kernel for 64 x 64 blocks and wide column tiles (AsyncSparse
// paper, Sections III-A to III-C; the dense blocks of a block row are a
// sequence of micro-GEMMs over gathered 64-row slices of B).  Built without
// forcing MFMA accumulators into ordinary VGPRs: at one wave per SIMD the
// accumulators live in the accumulation registers and the ordinary ones hold a
// deep ring of B loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace wspmm {

// BCSR with 64 x 64 blocks, one work-group of NW waves x 128 columns per CU.
// The work-group walks the half-blocks (32 k rows) of its block row; every
// wave keeps D half-blocks of B rows in flight in a ring of D+1 register
// stages (its 64 x 128 accumulators sit in the accumulation registers, which
// leaves the ordinary registers to the ring at one wave per SIMD).  The A
// block is loaded once per work-group, one block ahead, into one of two padded
// LDS buffers; the block-column indices of the block row are read once into a
// register (lane i holds block i, at most 64 blocks per row).  All loads are
// unconditional: half-blocks past the end read zeros.
template <int AB, int NW, int D>
__global__ __launch_bounds__(NW * 64, 1) void bcsr64_ring_kernel(TileParams p)
{
    constexpr int R = 64, BC = 64, MT = 4, V = 8, DW = 4;
    constexpr int Q = D + 1;                       // ring stages; even, so blocks align
    static_assert(Q % 2 == 0, "the ring must hold whole blocks");
    // A block q+AH is loaded at the start of block q, ahead of every B stage
    // still in flight when it is stored to LDS at the end of block q+AH-1, so
    // that wait never drains the ring; NA register copies rotate.
    constexpr int AH = 1 + (D - 1) / 2;
    constexpr int NA = Q / 2;                      // blocks per ring iteration
    static_assert(NA == AH, "one A register copy per block of an iteration");
    constexpr int NT = NW * 64;
    constexpr int STRIDE = BC * 2 + 16;            // padded LDS row: conflict-free b128 reads
    constexpr int ABUF = R * STRIDE;
    constexpr int CPT = R * BC / 8 / NT;           // 16-byte chunks per thread per block
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * ABUF];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;

    int64_t item, ctile;
    tile_of(p.n_items, p.n_items * p.n_col_tiles, p.order, item, ctile);
    const int64_t blk0 = p.row_ptr[item];
    const int nblk = p.row_ptr[item + 1] - (int)blk0;   // <= 64 (the plan checks)
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

    // block columns of this block row: lane i holds block i
    const __amdgpu_buffer_rsrc_t rJ = make_rsrc(p.col_idx + blk0, (uint32_t)nblk * 4u);
    const uint32_t vcols = __builtin_amdgcn_raw_buffer_load_b32(rJ, (uint32_t)lane * 4u, 0, 0);
    auto block_col = [&](int q) -> uint32_t {  // q wave-uniform; past the end: no block
        return q < nblk ? (uint32_t)__builtin_amdgcn_readlane((int)vcols, q & 63) : 0xFFFFFFFFu;
    };

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
    // B rows of half-block h: block column J of block h/2, rows 32*(h%2) + 8g + j
    auto issue_b = [&](int h, BStage<DW> &st) {
        const uint32_t J = block_col(h >> 1);
        const bool jv = J < nbc;
        const uint32_t r0 = (jv ? J : 0u) * BC + (uint32_t)(h & 1) * 32 + 8 * g;
        const uint32_t base = __umul24(r0, ldb2) + lane_col_bytes;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            buf_load<DW>(rB, (jv & (r0 + j < k32)) ? base + (uint32_t)j * ldb2 : kOOB, st.b[j]);
    };
    auto compute = [&](const BStage<DW> &st, int buf, int half) {
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

    const int nh = 2 * nblk;
    if (nh > 0) {
        u32x4_t areg[NA][CPT];   // areg[q % NA]: A block q between its load and its LDS store
        BStage<DW> st[Q];
        load_a(0, areg[0]);
        store_a(0, areg[0]);
#pragma unroll
        for (int q = 1; q < AH; ++q)
            load_a(q, areg[q % NA]);
#pragma unroll
        for (int u = 0; u < D; ++u)
            issue_b(u, st[u]);
        lds_barrier();
        for (int h0 = 0; h0 < nh; h0 += Q) {   // h0 / 2 is a multiple of NA
#pragma unroll
            for (int u = 0; u < Q; ++u) {
                const int h = h0 + u;
                const int b = u >> 1;             // block of the iteration
                __builtin_amdgcn_sched_barrier(0);
                issue_b(h + D, st[(u + D) % Q]);
                if ((u & 1) == 0)
                    load_a((h >> 1) + AH, areg[(b + AH) % NA]);  // zeros past the end
                __builtin_amdgcn_sched_barrier(0);
                compute(st[u], (h >> 1) & 1, u & 1);
                if (u & 1) {
                    __builtin_amdgcn_sched_barrier(0);
                    store_a(((h >> 1) + 1) & 1, areg[(b + 1) % NA]);
                    lds_barrier();
                }
            }
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

template <int D>
static void launch_ring_d(int ab, const TileParams &p, hipStream_t stream)
{
    dim3 grid((unsigned)(p.n_items * p.n_col_tiles));
    if (ab == SPMM_FP16)
        hipLaunchKernelGGL((bcsr64_ring_kernel<SPMM_FP16, 4, D>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((bcsr64_ring_kernel<SPMM_BF16, 4, D>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_bcsr64_ring(int ab, int depth, const TileParams &p, hipStream_t stream)
{
    if (depth == 3)
        launch_ring_d<3>(ab, p, stream);
    else
        launch_ring_d<5>(ab, p, stream);
    return hipGetLastError();
}

}  // namespace wspmm

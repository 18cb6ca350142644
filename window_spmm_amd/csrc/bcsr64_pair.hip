// BCSR SpMM with 64 x 64 blocks and short block rows (at most 6 blocks), wide
// N: the block row's A blocks held in registers by a pair of waves.
//
// The computation is the paper's BCSR product (Section III-A: one work-group
// per block row and column tile, each stored block multiplied with the B tile
// of its block column, accumulated in fp32; Section III-C: the staged B
// pipeline).  What differs is the dataflow, chosen for the MI355X cache sizes.
//
// Where the time went before.  With 512-column tiles per work-group (four
// waves of 128 columns) the 64 work-groups resident on one XCD read a B column
// slice of 3584 x 512 x 2 bytes = 3.7 MB at a time, nearly the whole 4 MB L2 of
// the XCD, so B rows were fetched from memory about 13 times over.
//
// Here a work-group is two waves that together own one block row and sweep a
// range of 128-column strips.  Wave w keeps blocks w, w + 2, w + 4 of the row in
// registers for the whole sweep (96 VGPRs: 64 rows x 3 blocks x 64 columns of
// bf16 split over 64 lanes), so A is read once per (block row, range) and never
// through LDS; the wave multiplies its blocks with the matching 64 x 128 B
// tiles, and the two partial 64 x 128 tiles are added through LDS at the end of
// each strip: each wave writes the half of its partial tile the other wave
// stores, one barrier, each adds and stores 32 rows.  Two work-groups per CU
// (one wave per SIMD) put 64 block rows on an XCD, all sweeping the same
// 128-column strip: the B slice they share is 3584 x 128 x 2 = 0.9 MB, a
// quarter of the XCD's L2.
//
// MFMA mapping as in the other kernels (v_mfma_f32_16x16x32, lane 16g + i holds
// A[row i][8 k from 8g] and B[8 k from 8g][column i]; B rows are loaded 8
// columns per lane and transposed in registers).  Each wave keeps two k-steps
// of B loads in flight in a ring of three register stages; the ring runs on
// across strip boundaries, so the next strip's first loads overlap this
// strip's reduction and stores.  Launch order deals work-groups to the XCDs in
// turn; XCD x runs the column ranges x, x + 8, ... and, inside a range, the
// block rows in order, so its resident work-groups start together and move
// through the same strips at the same pace.
//
// Measured on the 18944 x 3584 gate_proj weight at N = 65536 (6 blocks per block
// row), against the sweep kernel on the same box: memory-side reads fall from
// 6.8 to 3.8 GB per launch (L2 hit rate 0.56 -> 0.69, mean L1-miss latency 415
// -> 273 cycles), yet the launch takes 1.51 ms against 1.40 ms.  Timing-only
// copies locate the cost: without any B load the kernel runs in 0.74 ms, and
// the B loads add their own time instead of overlapping it (a deeper ring, B
// kept in L2, or B loaded straight into LDS change it by under 10 %), because
// the vector-memory data path that carries every B byte to the 64 rows it
// feeds is the busy unit (its texture data unit is 83 % busy, the sweep
// kernel's 95 %, at the 1.6-1.8 GHz the chip holds under this load).  The
// plan therefore keeps the sweep kernel for these
// shapes; this kernel remains an option for callers and the tile sweep.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace wspmm {

namespace {

constexpr int kPairBlocksPerWave = 3;              // blocks of a block row per wave
constexpr int kPairSteps = 2 * kPairBlocksPerWave; // 32-deep k-steps per strip per wave
constexpr int kPairStages = 3;                     // ring stages (two steps in flight)
static_assert(kPairSteps % kPairStages == 0, "a strip's steps fill whole ring turns");
// LDS: two strip parities x two waves x a 32 x 128 fp32 half tile
constexpr int kPairHalfFloats = 32 * 128;
constexpr size_t kPairLdsBytes = 2 * 2 * kPairHalfFloats * sizeof(float);

}  // namespace

size_t pair_lds_bytes() { return kPairLdsBytes; }

template <int AB>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bcsr64_pair_kernel(TileParams p)
{
    constexpr int R = 64, BC = 64, MT = 4, V = 8, DW = 4;
    constexpr int NB = kPairBlocksPerWave, S = kPairSteps, Q = kPairStages;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    f32x4_t *const red = reinterpret_cast<f32x4_t *>(smem);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;

    // work-group -> (column range, block row): XCD x runs ranges x, x + 8, ...
    const uint32_t xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const uint32_t h = local / (uint32_t)p.n_items;
    const uint32_t item = __builtin_amdgcn_readfirstlane(local - h * (uint32_t)p.n_items);
    const int64_t t_begin = (int64_t)(h * 8 + xcd) * p.range_tiles;
    const int64_t t_end = t_begin + p.range_tiles < p.n_col_tiles ? t_begin + p.range_tiles
                                                                  : p.n_col_tiles;
    if (t_begin >= t_end)
        return;  // the whole work-group
    const int ntiles = (int)(t_end - t_begin);
    const int64_t blk0 = p.row_ptr[item];
    const int nblk = p.row_ptr[item + 1] - (int)blk0;  // <= 2 * NB (the plan checks)
    const int64_t row0 = (int64_t)item * R;

    // this wave's blocks: q = wave + 2j, j < NB; block columns through lane j
    const __amdgpu_buffer_rsrc_t rJ = make_rsrc(p.col_idx + blk0, (uint32_t)nblk * 4u);
    const uint32_t vcols = __builtin_amdgcn_raw_buffer_load_b32(
        rJ, lane < NB ? (uint32_t)(wave + 2 * lane) * 4u : kOOB, 0, 0);

    // A fragments of the wave's blocks: a[j][hf][mt] = rows 16mt + li,
    // k = 32hf + 8g .. +7 of block wave + 2j (zeros past the row's end)
    u32x4_t a[NB][2][MT];
    {
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(p.A + blk0 * R * BC, (uint32_t)((int64_t)nblk * R * BC * 2));
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int q = wave + 2 * j;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t off = (((uint32_t)q * R + 16 * mt + li) * BC + 32 * hf + 8 * g) * 2u;
                    a[j][hf][mt] = __builtin_amdgcn_raw_buffer_load_b128(rA, q < nblk ? (int)off : (int)kOOB,
                                                                         0, 0);
                }
        }
    }

    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B, (uint32_t)p.b_bytes);
    const uint32_t ldb2 = (uint32_t)p.ldb * 2;
    const uint32_t k32 = (uint32_t)p.k;
    const uint32_t nbc = (uint32_t)((p.k + BC - 1) / BC);
    const uint32_t lane_col = (uint32_t)(li * V);           // this lane's first column of a strip
    const int64_t col_first = t_begin * 128 + lane_col;
    const int esz = p.c_dtype == SPMM_FP32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc((uint8_t *)p.C + row0 * p.ldc * esz, (uint32_t)(R * p.ldc * esz));

    // B rows of step s (block wave + 2(s/2), half s%2) of strip t: rows J*64 +
    // 32(s%2) + 8g + j, 8 columns from this lane's; strip ntiles loads nothing
    auto issue = [&](int t, int s, BStage<DW> &st) {
        const int j = s >> 1, hf = s & 1;
        const uint32_t J = (uint32_t)__builtin_amdgcn_readlane((int)vcols, j);
        const bool jv = (t < ntiles) & (wave + 2 * j < nblk) & (J < nbc);
        const uint32_t r0 = (jv ? J : 0u) * BC + (uint32_t)hf * 32 + 8 * g;
        const uint32_t base = r0 * ldb2 + (uint32_t)col_first * 2u + (uint32_t)t * 256u;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            buf_load<DW>(rB, (jv & (r0 + jj < k32)) ? base + (uint32_t)jj * ldb2 : kOOB, st.b[jj]);
    };

    f32x4_t acc[MT][V];
    auto compute = [&](const BStage<DW> &st, int s) {
        const int j = s >> 1, hf = s & 1;
#pragma unroll
        for (int c = 0; c < V; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t bf;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                bf[qq] = __builtin_amdgcn_perm(st.b[2 * qq + 1][c >> 1], st.b[2 * qq][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(a[j][hf][mt], bf, acc[mt][c]);
        }
    };

    // End of strip t: wave w stores rows 32w .. 32w + 31 (slices mt = 2w, 2w + 1)
    // and hands the other wave the slices it stores.  LDS slot of (parity, writer
    // wave, slice m2, column group c, lane): f32x4 index ((par*2 + wave)*2 + m2)*8 + c,
    // times 64 lanes -- every b128 access covers 1 KB contiguously.  W is the
    // wave as a compile-time constant (the accumulator slices are then
    // addressed with constant indices and stay in registers), DT the C type.
    auto finish = [&](int t, auto W, auto DTc) {
        constexpr int w = decltype(W)::value;
        constexpr int DT = decltype(DTc)::value;
        constexpr int esz_c = DT == SPMM_FP32 ? 4 : 2;
        const int par = t & 1;
        constexpr int give = 2 * (1 - w);  // first slice the partner stores
        constexpr int keep = 2 * w;
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int c = 0; c < V; ++c)
                red[((((par * 2 + w) * 2 + m2) * V + c) << 6) + lane] = acc[give + m2][c];
        lds_barrier();
        const int64_t ncol = col_first + (int64_t)t * 128;
        const bool col_ok = ncol < p.N;
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            // one slice at a time: add the partner's partial, then store its 16 rows
#pragma unroll
            for (int c = 0; c < V; ++c)
                acc[keep + m2][c] += red[((((par * 2 + (1 - w)) * 2 + m2) * V + c) << 6) + lane];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int r = (keep + m2) * 16 + 4 * g + qq;
                const bool ok = col_ok & (row0 + r < p.m);
                const uint32_t off = ok ? (uint32_t)((r * p.ldc + ncol) * esz_c) : kOOB;
                if constexpr (DT == SPMM_FP32) {
#pragma unroll
                    for (int c = 0; c < V; c += 4) {
                        const f32x4_t v = {acc[keep + m2][c][qq], acc[keep + m2][c + 1][qq],
                                           acc[keep + m2][c + 2][qq], acc[keep + m2][c + 3][qq]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rC,
                                                               (int)(off == kOOB ? kOOB : off + 4 * c), 0, kNT);
                    }
                } else {
                    u32x4_t packed;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        packed[c] = pack2(DT, acc[keep + m2][2 * c][qq], acc[keep + m2][2 * c + 1][qq]);
                    __builtin_amdgcn_raw_buffer_store_b128(packed, rC, (int)off, 0, kNT);

                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto finish_w = [&](int t, auto W) {
        if (p.c_dtype == SPMM_FP32)
            finish(t, W, std::integral_constant<int, SPMM_FP32>{});
        else if (p.c_dtype == SPMM_BF16)
            finish(t, W, std::integral_constant<int, SPMM_BF16>{});
        else
            finish(t, W, std::integral_constant<int, SPMM_FP16>{});
    };

    BStage<DW> st[Q];
#pragma unroll
    for (int u = 0; u < Q - 1; ++u)
        issue(0, u, st[u]);
    for (int t = 0; t < ntiles; ++t) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int c = 0; c < V; ++c)
                acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // step s + Q - 1 (of this strip or the next) into the stage step s - 1 used
            const int s2 = s + Q - 1;
            __builtin_amdgcn_sched_barrier(0);
            issue(s2 < S ? t : t + 1, s2 < S ? s2 : s2 - S, st[s2 % Q]);
            compute(st[s % Q], s);
            // one B load per four MFMAs: spreading the loads over the step keeps
            // the address unit fed without holding the wave (measured: 3 %)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one B load
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // four MFMAs
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (wave == 0)
            finish_w(t, std::integral_constant<int, 0>{});
        else
            finish_w(t, std::integral_constant<int, 1>{});
    }
}

template __global__ void bcsr64_pair_kernel<SPMM_FP16>(TileParams);
template __global__ void bcsr64_pair_kernel<SPMM_BF16>(TileParams);

static const void *pair_fn(int ab)
{
    return ab == SPMM_FP16 ? reinterpret_cast<const void *>(bcsr64_pair_kernel<SPMM_FP16>)
                           : reinterpret_cast<const void *>(bcsr64_pair_kernel<SPMM_BF16>);
}

hipError_t launch_bcsr64_pair(int ab, const TileParams &p, hipStream_t stream)
{
    TileParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(pair_fn(ab), dim3((unsigned)(p.n_items * p.n_ranges)), dim3(128), args,
                           kPairLdsBytes, stream);
}

int pair_blocks_per_cu(int ab)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pair_fn(ab), 128, kPairLdsBytes) != hipSuccess)
        return 0;
    return n;
}

}  // namespace wspmm

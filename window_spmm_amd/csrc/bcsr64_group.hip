// BCSR SpMM with 64 x 64 blocks and short block rows (at most 6 blocks), wide N:
// groups of four block rows that share B tiles through an LDS ring, with
// producer and consumer roles synchronised by LDS counters (the paper's staged
// pipeline, Section III-B / III-C and Fig. 4, rebuilt for gfx950).
//
// Why.  Each B element a 64-row block brings into a CU feeds 64 rows, and on the
// Qwen2.5-7B gate_proj shape (6 random blocks out of 56 per block row) moving B
// through the vector-memory path is what bounds the one-block-row-per-work-group
// kernels: without their B loads they run in about half the time.  Block rows
// that share block columns can share those B tiles.  The plan groups block rows
// four at a time, greedily by shared block columns (on that shape a group needs
// 1.7 times fewer distinct B tiles than its rows hold), and a work-group runs one
// group: its union of block columns is streamed through LDS once per 64-column
// strip, and every block row that holds a block column multiplies its A block
// with the staged tile.
//
// Roles.  A work-group is four waves, one per block row of the group (one wave
// per SIMD); wave w keeps its row's A blocks in registers for the whole sweep.
// The tiles of a strip form a sequence of items, two per union column (its two
// 32-row halves), strips one after the other.  Item x goes into LDS slot x mod
// S.  Wave x mod 4 produces item x: it waits until every consumer of the slot's
// previous item (x - S) is done with it, clears the slot's done counter and
// loads the tile (32 rows x 64 columns, 16 bytes per lane in four loads) into
// registers; later it writes the tile into the slot and then x into the slot's
// full word.  (The tiles go through registers rather than direct-to-LDS loads:
// the compiler cannot tell a direct-to-LDS load from the LDS reads of other
// slots and would make every LDS read wait for all of them.)  Each wave
// consumes the items of its own block columns, in order: it waits until the
// slot's full word reads x, reads the tile, runs its MFMAs and adds one to the
// slot's done counter.
//
// Progress.  A wave produces its items (two at a time, x and x + 4) up to 20
// beyond the item it is about to consume (and, at the end of a strip, up to 20
// beyond the strip), never more: with 24 slots every wait then depends only on
// operations of lower item index,
// so no wait can close a cycle.  Before any wait a wave publishes the items it
// has loaded (waits for its loads, then writes their full words), so a wave that
// waits never holds back an item another wave needs; otherwise a wave writes a
// pair out at its next production.  Every wait is a bounded
// spin: a fault in these rules would give wrong numbers, never a hang.
//
// LDS layout of an item (4 KB): chunk (row r = 8g + j, 16-byte column chunk q) at
// ((4j + g) * 8 + q) * 16, which the producer writes as 1 KB runs (lane l of its
// i-th load holds bytes 1024 i + 16 l .. +15) and a consumer reads conflict-free: for each j its 64 lanes read 512 contiguous
// bytes (8 bytes each: columns 4i .. 4i + 3 of row 8g + j for lane 16g + i).
//
// Measured on the 18944 x 3584 gate_proj weight at N = 65536: 2.49 ms per
// launch, against 1.41 ms for the sweep kernel on the same box, although it
// loads 1.7 times fewer B tiles.  A timing copy with every wait removed (wrong
// results, same instruction stream otherwise) takes 2.45 ms, and one that
// publishes each item as soon as it is loaded 2.71 ms: the synchronisation is
// not where the time goes.  With one wave per SIMD nothing hides the latency
// of each pair's loads and of every item's trip through LDS; the sweep kernel
// keeps two k-steps of loads in flight per wave and no LDS round trip between
// load and MFMA.  The plan therefore never picks this kernel; it stays an
// option for callers and the tile sweep.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace wspmm {

namespace {

constexpr int kG = kGroupRows;                  // block rows per group (waves per work-group)
constexpr int kNB = kGroupMaxBlocks;            // blocks per block row, at most
constexpr int kMaxU = kG * kNB;                 // union columns per group, at most
constexpr int kSlots = 24;                      // LDS ring slots
constexpr int kAhead = 16;                      // production lookahead
// a pair's second item lies kGroupRows beyond the lookahead: still below the ring size
static_assert(kAhead + kGroupRows < kSlots, "production lookahead must stay below the ring size");
constexpr int kItemBytes = 32 * 64 * 2;         // 32 rows x 64 columns of 16-bit codes
constexpr int kRingBytes = kSlots * kItemBytes;
constexpr int kSpinLimit = 1 << 22;             // polls before a wait gives up
// LDS: ring | full words | done counters | union columns | consumer counts
constexpr size_t kGroupLdsBytes = kRingBytes + (2 * kSlots + 2 * kMaxU) * sizeof(int32_t);

}  // namespace

size_t group_lds_bytes() { return kGroupLdsBytes; }

template <int AB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bcsr64_group_kernel(TileParams p, const int32_t *__restrict__ gtab)
{
    constexpr int R = 64, BC = 64, MT = 4, V = 4, DW = 2;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int32_t *const full = reinterpret_cast<int32_t *>(smem + kRingBytes);
    int32_t *const done = full + kSlots;
    int32_t *const ucol = done + kSlots;
    int32_t *const ucnt = ucol + kMaxU;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;

    // work-group -> (column range, group): XCD x runs ranges x, x + 8, ...
    const uint32_t xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const uint32_t hr = local / (uint32_t)p.n_items;
    const uint32_t grp = __builtin_amdgcn_readfirstlane(local - hr * (uint32_t)p.n_items);
    const int64_t t_begin = (int64_t)(hr * 8 + xcd) * p.range_tiles;
    const int64_t t_end = t_begin + p.range_tiles < p.n_col_tiles ? t_begin + p.range_tiles
                                                                  : p.n_col_tiles;
    if (t_begin >= t_end)
        return;  // the whole work-group
    const int ntiles = (int)(t_end - t_begin);

    // group table: rows[4], nU, U[kMaxU], cnt[kMaxU], pos[4][kNB]
    const int32_t *tab = gtab + (int64_t)grp * kGroupTableInts;
    const int nU = tab[kG];
    if (threadIdx.x < kMaxU) {
        ucol[threadIdx.x] = tab[kG + 1 + threadIdx.x];
        ucnt[threadIdx.x] = tab[kG + 1 + kMaxU + threadIdx.x];
    }
    if (threadIdx.x < kSlots) {
        full[threadIdx.x] = -1;
        done[threadIdx.x] = 0;
    }
    const int row = tab[wave];                              // -1: no block row for this wave
    const int64_t blk0 = row >= 0 ? p.row_ptr[row] : 0;
    const int nblk = row >= 0 ? p.row_ptr[row + 1] - (int)blk0 : 0;
    // union position of this wave's block q: lane q holds it
    const int32_t vpos = tab[kG + 1 + 2 * kMaxU + wave * kNB + (lane < kNB ? lane : 0)];

    // A fragments: a[q][h][mt] = rows 16mt + li, k = 32h + 8g .. +7 of block q
    u32x4_t a[kNB][2][MT];
    {
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(p.A + blk0 * R * BC, (uint32_t)((int64_t)nblk * R * BC * 2));
#pragma unroll
        for (int q = 0; q < kNB; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t off = (((uint32_t)q * R + 16 * mt + li) * BC + 32 * h + 8 * g) * 2u;
                    a[q][h][mt] = __builtin_amdgcn_raw_buffer_load_b128(rA, q < nblk ? (int)off : (int)kOOB,
                                                                        0, 0);
                }
    }
    __syncthreads();

    const int ips = 2 * nU;                                 // items per strip
    const int total = ntiles * ips;
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B, (uint32_t)p.b_bytes);
    const uint32_t ldb2 = (uint32_t)p.ldb * 2;
    const uint32_t k32 = (uint32_t)p.k;
    const uint32_t nbc = (uint32_t)((p.k + BC - 1) / BC);
    const int64_t strip0 = t_begin * 64;                    // first column of the range
    const int esz = p.c_dtype == SPMM_FP32 ? 4 : 2;
    const int64_t row0 = (int64_t)(row >= 0 ? row : 0) * R;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc((uint8_t *)p.C + row0 * p.ldc * esz, (uint32_t)(R * p.ldc * esz));

    // This lane's part of any item: instruction i writes bytes [1024 i, 1024 i +
    // 1024) of the slot, lane l bytes 16 l .. 16 l + 15 of that run, which hold
    // chunk q = f % 8 of row 8 * ((f / 8) % 4) + f / 32, f = 64 i + l.
    uint32_t lane_row[4], lane_col[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f = 64 * i + lane;
        lane_row[i] = (uint32_t)(8 * ((f >> 3) & 3) + (f >> 5));
        lane_col[i] = (uint32_t)(8 * (f & 7));
    }

    int next_prod = wave;       // next item this wave produces
    // This wave produces its items in pairs (x, x + 4): a pair's eight loads land
    // in two fixed register buffers, and the pair is written to its slots (and
    // their full words set) at the wave's next production, before any wait, or at
    // the end -- by then the loads have had a production interval to arrive.
    u32x4_t stg_a[4], stg_b[4];
    int pend_a = -1, pend_b = -1;   // items the buffers hold (-1: none)

    // bounded spin until *w == want (workgroup-scope acquire)
    auto spin_until = [&](const int32_t *w, int want) {
        for (int it = 0; it < kSpinLimit; ++it) {
            if (__hip_atomic_load(w, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == want)
                return;
            __builtin_amdgcn_s_sleep(1);
        }
    };
    // write a staged item into its slot, then set the slot's full word
    auto write_item = [&](int x, const u32x4_t (&v)[4]) {
        uint8_t *dst = smem + (x % kSlots) * kItemBytes + lane * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4_t *>(dst + i * 1024) = v[i];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the tile is in LDS
        if (lane == 0)
            __hip_atomic_store(&full[x % kSlots], x, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto publish = [&]() {
        if (pend_a >= 0)
            write_item(pend_a, stg_a);
        if (pend_b >= 0)
            write_item(pend_b, stg_b);
        pend_a = pend_b = -1;
    };
    // loads of item x into a staging buffer
    auto load_item = [&](int x, u32x4_t (&v)[4]) {
        const int t = x / ips, r = x - t * ips;
        const uint32_t J = (uint32_t)ucol[r >> 1];
        const int h = r & 1;
        const bool jv = J < nbc;
        const uint32_t rbase = (jv ? J : 0u) * BC + 32u * h;
        const uint32_t cbase = (uint32_t)(strip0 + (int64_t)t * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t rr = rbase + lane_row[i];
            const uint32_t off = (jv & (rr < k32)) ? rr * ldb2 + (cbase + lane_col[i]) * 2u : kOOB;
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)off, 0, 0);
        }
    };
    // before item x goes into its slot, every consumer of the slot's previous
    // item must be done with it; then the slot's done counter restarts
    auto claim_slot = [&](int x) {
        const int slot = x % kSlots;
        if (x >= kSlots) {
            const int prev = x - kSlots;
            const int want = ucnt[(prev % ips) >> 1];
            if (__hip_atomic_load(&done[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != want) {
                publish();
                spin_until(&done[slot], want);
            }
        }
        if (lane == 0)
            __hip_atomic_store(&done[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // produce this wave's items (in pairs) while the pair's first item is at most
    // `upto` (items beyond the last do not exist)
    auto produce_upto = [&](int upto) {
        if (upto >= total)
            upto = total - 1;
        while (next_prod <= upto) {
            const int x = next_prod, y = next_prod + kG;
            claim_slot(x);
            if (y < total)
                claim_slot(y);
            publish();
            load_item(x, stg_a);
            pend_a = x;
            if (y < total) {
                load_item(y, stg_b);
                pend_b = y;
            }
            next_prod += 2 * kG;
        }
    };

    f32x4_t acc[MT][V];
    // consume item x with the A fragments of one block half
    auto consume = [&](int x, const u32x4_t (&af)[MT]) {
        const int slot = x % kSlots;
        if (__hip_atomic_load(&full[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != x) {
            publish();
            spin_until(&full[slot], x);
        }
        const uint8_t *base = smem + slot * kItemBytes + li * 8;
        uint32_t b[8][DW];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x2_t v = *reinterpret_cast<const u32x2_t *>(base + (4 * j + g) * 128);
            b[j][0] = v[0];
            b[j][1] = v[1];
        }
#pragma unroll
        for (int c = 0; c < V; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t bf;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                bf[qq] = __builtin_amdgcn_perm(b[2 * qq + 1][c >> 1], b[2 * qq][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(af[mt], bf, acc[mt][c]);
        }
        // the tile has been read (the MFMAs used it): one more consumer done
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        if (lane == 0)
            __hip_atomic_fetch_add(&done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    // stores strip t of this wave's block row as DT (non-temporal)
    auto store = [&](int t, auto DTc) {
        constexpr int DT = decltype(DTc)::value;
        constexpr int esz_c = DT == SPMM_FP32 ? 4 : 2;
        const int64_t ncol = strip0 + (int64_t)t * 64 + li * V;
        const bool col_ok = ncol < p.N;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int r = mt * 16 + 4 * g + qq;
                const bool ok = col_ok & (row0 + r < p.m);
                const uint32_t off = ok ? (uint32_t)((r * p.ldc + ncol) * esz_c) : kOOB;
                if constexpr (DT == SPMM_FP32) {
                    const f32x4_t v = {acc[mt][0][qq], acc[mt][1][qq], acc[mt][2][qq], acc[mt][3][qq]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rC, (int)off, 0, kNT);
                } else {
                    const u32x2_t v = {pack2(DT, acc[mt][0][qq], acc[mt][1][qq]),
                                       pack2(DT, acc[mt][2][qq], acc[mt][3][qq])};
                    __builtin_amdgcn_raw_buffer_store_b64(v, rC, (int)off, 0, kNT);
                }
            }
    };

    for (int t = 0; t < ntiles; ++t) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int c = 0; c < V; ++c)
                acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < kNB; ++q) {
            const int u = __builtin_amdgcn_readlane(vpos, q);  // -1: no union column
            if (q < nblk && u >= 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int x = t * ips + 2 * u + h;
                    produce_upto(x + kAhead);
                    consume(x, a[q][h]);
                }
            }
        }
        produce_upto((t + 1) * ips - 1 + kAhead);
        if (row >= 0) {
            if (p.c_dtype == SPMM_FP32)
                store(t, std::integral_constant<int, SPMM_FP32>{});
            else if (p.c_dtype == SPMM_BF16)
                store(t, std::integral_constant<int, SPMM_BF16>{});
            else
                store(t, std::integral_constant<int, SPMM_FP16>{});
        }
    }
    produce_upto(total - 1);
    publish();
}

template __global__ void bcsr64_group_kernel<SPMM_FP16>(TileParams, const int32_t *);
template __global__ void bcsr64_group_kernel<SPMM_BF16>(TileParams, const int32_t *);

static const void *group_fn(int ab)
{
    return ab == SPMM_FP16 ? reinterpret_cast<const void *>(bcsr64_group_kernel<SPMM_FP16>)
                           : reinterpret_cast<const void *>(bcsr64_group_kernel<SPMM_BF16>);
}

hipError_t launch_bcsr64_group(int ab, const TileParams &p, const int32_t *gtab, hipStream_t stream)
{
    TileParams arg = p;
    const int32_t *t = gtab;
    void *args[] = {&arg, &t};
    return hipLaunchKernel(group_fn(ab), dim3((unsigned)(p.n_items * p.n_ranges)), dim3(256), args,
                           kGroupLdsBytes, stream);
}

int group_blocks_per_cu(int ab)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, group_fn(ab), 256, kGroupLdsBytes) != hipSuccess)
        return 0;
    return n;
}

}  // namespace wspmm

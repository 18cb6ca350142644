// gfx950 kernels for BCSR and WCSR SpMM (AsyncSparse paper, Sections III-A..III-C).
//
// Both formats reduce to the same per-tile computation.  A work-group tile owns
// R consecutive rows of C (a BCSR block row or a WCSR window, R = b_row) and a
// BN-wide slice of its columns.  Along the reduction the tile walks a "packed"
// column axis k':
//   BCSR  k' = q*b_col + kk  for the q-th stored block of the block row:
//         A(r, k') = blocks[q][r][kk],  B row = block_col_idx[q]*b_col + kk
//   WCSR  k' = p, a packed column of the window:
//         A(r, p)  = window tile[r][p],  B row = window_col_idx[p]  (-1 = pad)
// so the tile is a dense R x K' x BN product whose B operand is a row gather.
//
// MFMA mapping (v_mfma_f32_16x16x32_{f16,bf16}, wave64).  Lane l = 16*g + i
// supplies A[row i][k-group g] (8 consecutive k') and B[k-group g][column i];
// accumulator element q of lane l is D[4*g + q][i].  The k' rows of B are
// N-contiguous in memory while MFMA wants 8 consecutive k per lane, so every
// lane loads V consecutive columns of 8 gathered rows (one 2V-byte load per
// row) and transposes the 8 x V block in registers (v_perm_b32).  That gives
// the lane the B operand of V different 16x16 output tiles: in tile c, MFMA
// column i stands for C column  n_wave + i*V + c.  The accumulators of one lane
// therefore hold V adjacent columns of each of its rows, which the epilogue
// stores with one wide store per row.
//
// Waves of a work-group split the tile's columns (waves_n, each 16*V wide) and
// the reduction (waves_k, interleaved 32-wide k' steps); the waves_k partial
// sums are added in a fixed order through LDS, so results are deterministic.
// WCSR tasks that cover only part of a long window write fp32 partial tiles to
// a workspace slot; wcsr_merge adds the slots of a window in slot order and
// rounds once (this replaces the paper's atomicAdd merge, Section III-C).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace wspmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int AB>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c)
{
    if constexpr (AB == SPMM_FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bfloat16 code, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> binary16 code (hardware conversion, round to nearest even).
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Loads DW dwords (DW = 1, 2, 4) from a naturally aligned address.
template <int DW>
__device__ __forceinline__ void load_dw(const uint16_t *p, uint32_t *out)
{
    if constexpr (DW == 4) {
        u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (DW == 2) {
        u32x2_t v = *reinterpret_cast<const u32x2_t *>(p);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = *reinterpret_cast<const uint32_t *>(p);
    }
}

// Stores V consecutive results of one row as c_dtype.
template <int V>
__device__ __forceinline__ void store_row(void *base, int64_t elem, int c_dtype, const float *v)
{
    if (c_dtype == SPMM_FP32) {
        float *d = reinterpret_cast<float *>(base) + elem;
#pragma unroll
        for (int c = 0; c < V; c += 4) {
            if constexpr (V >= 4) {
                f32x4_t x = {v[c], v[c + 1], v[c + 2], v[c + 3]};
                *reinterpret_cast<f32x4_t *>(d + c) = x;
            }
        }
        if constexpr (V == 2) {
            typedef float f32x2_t __attribute__((ext_vector_type(2)));
            f32x2_t x = {v[0], v[1]};
            *reinterpret_cast<f32x2_t *>(d) = x;
        }
    } else {
        uint32_t w[V / 2];
#pragma unroll
        for (int c = 0; c < V; c += 2) {
            uint32_t lo = c_dtype == SPMM_BF16 ? f32_to_bf16(v[c]) : f32_to_f16(v[c]);
            uint32_t hi = c_dtype == SPMM_BF16 ? f32_to_bf16(v[c + 1]) : f32_to_f16(v[c + 1]);
            w[c / 2] = lo | (hi << 16);
        }
        uint16_t *d = reinterpret_cast<uint16_t *>(base) + elem;
        if constexpr (V == 8) {
            u32x4_t x = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4_t *>(d) = x;
        } else if constexpr (V == 4) {
            u32x2_t x = {w[0], w[1]};
            *reinterpret_cast<u32x2_t *>(d) = x;
        } else {
            *reinterpret_cast<uint32_t *>(d) = w[0];
        }
    }
}

template <int FMT, int R, int V, int AB>
__global__ __launch_bounds__(512) void spmm_tile_kernel(TileParams p)
{
    constexpr int MT = R / 16;  // 16-row MFMA tiles per work-group tile
    constexpr int DW = V / 2;   // dwords of one gathered row segment per lane
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % p.waves_n;
    const int wk = wave / p.waves_n;
    const int g = lane >> 4;
    const int li = lane & 15;

    // ---- work item -------------------------------------------------------
    int64_t row0, kbegin, kend, a_base = 0, wcols = 0, blk0 = 0;
    int32_t slot = -1;
    if constexpr (FMT == 0) {
        const int64_t I = blockIdx.x;
        blk0 = p.row_ptr[I];
        row0 = I * R;
        kbegin = 0;
        kend = (int64_t)(p.row_ptr[I + 1] - blk0) * p.b_col;
    } else {
        const int4 t = p.tasks[blockIdx.x];
        const int64_t w = t.x;
        row0 = w * R;
        kbegin = t.y;
        kend = t.z;
        slot = t.w;
        a_base = p.row_ptr[w];                  // packed column where the window starts
        wcols = p.row_ptr[w + 1] - a_base;      // window width W
    }
    const int64_t ncol = (int64_t)blockIdx.y * p.tile_cols + wn * 16 * V + li * V;
    const bool ncol_ok = ncol < p.N;

    f32x4_t acc[MT][V];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < V; ++c)
            acc[mt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = kbegin + 32 * wk; kb < kend; kb += 32 * p.waves_k) {
        const int64_t kg = kb + 8 * g;        // this lane's first k'
        const bool gvalid = kg < kend;

        // ---- B row of each of the 8 k' (index translation) ----
        int64_t brow[8];
        if constexpr (FMT == 0) {
            int64_t q = kg / p.b_col;
            int64_t kk = kg - q * p.b_col;
            int64_t J = gvalid ? (int64_t)p.col_idx[blk0 + q] : -1;
            int64_t r0 = J >= 0 ? J * p.b_col + kk : -1;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                brow[j] = r0 >= 0 ? r0 + j : -1;
        } else {
            if (gvalid) {
                const int4 *ip = reinterpret_cast<const int4 *>(p.col_idx + kg);
                int4 x0 = ip[0], x1 = ip[1];
                brow[0] = x0.x; brow[1] = x0.y; brow[2] = x0.z; brow[3] = x0.w;
                brow[4] = x1.x; brow[5] = x1.y; brow[6] = x1.z; brow[7] = x1.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    brow[j] = -1;
            }
        }

        // ---- gather V columns of the 8 B rows ----
        uint32_t bw[8][DW];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (ncol_ok && brow[j] >= 0 && brow[j] < p.k) {
                load_dw<DW>(p.B + brow[j] * p.ldb + ncol, bw[j]);
            } else {
#pragma unroll
                for (int d = 0; d < DW; ++d)
                    bw[j][d] = 0;
            }
        }

        // ---- A fragments: row li of each 16-row tile, 8 consecutive k' ----
        u32x4_t af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (gvalid) {
                int64_t off;
                if constexpr (FMT == 0) {
                    int64_t q = kg / p.b_col;
                    off = (blk0 + q) * (int64_t)(R * p.b_col) + (int64_t)(mt * 16 + li) * p.b_col +
                          (kg - q * p.b_col);
                } else {
                    off = R * a_base + (int64_t)(mt * 16 + li) * wcols + (kg - a_base);
                }
                af[mt] = *reinterpret_cast<const u32x4_t *>(p.A + off);
            } else {
                af[mt] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }

        // ---- transpose 8 rows x V columns into V operands of 8 k' each ----
#pragma unroll
        for (int c = 0; c < V; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t bf;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bf[q] = __builtin_amdgcn_perm(bw[2 * q + 1][c >> 1], bw[2 * q][c >> 1], sel);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][c] = mfma16x16x32<AB>(af[mt], bf, acc[mt][c]);
        }
    }

    // ---- fixed-order sum of the waves_k partial tiles through LDS ----
    if (p.waves_k > 1) {
        extern __shared__ float red[];  // [waves_n][MT*V*4][64]
        constexpr int NR = MT * V * 4;
        float *mine = red + (int64_t)wn * NR * 64 + lane;
        for (int s = p.waves_k - 1; s >= 1; --s) {
            if (wk == s) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int c = 0; c < V; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            mine[((mt * V + c) * 4 + q) * 64] = acc[mt][c][q];
            }
            __syncthreads();
            if (wk == 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int c = 0; c < V; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[mt][c][q] += mine[((mt * V + c) * 4 + q) * 64];
            }
            __syncthreads();
        }
        if (wk != 0)
            return;
    }

    // ---- epilogue: row 4g+q of each 16-row tile, V adjacent columns ----
    if (!ncol_ok)
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
            if (slot >= 0) {
                store_row<V>(p.partial, ((int64_t)slot * R + r) * p.N + ncol, SPMM_FP32, v);
            } else if (row0 + r < p.m) {
                store_row<V>(p.C, (row0 + r) * p.ldc + ncol, p.c_dtype, v);
            }
        }
    }
}

// One work-group per (merge record, chunk of 256*8 tile elements): adds the
// partial tiles of a split window in slot order and writes C once.
__global__ __launch_bounds__(256) void wcsr_merge_kernel(MergeParams p)
{
    const int3 mr = p.merges[blockIdx.x];
    const int64_t chunk = (int64_t)blockIdx.y * 256 + threadIdx.x;  // 8 columns each
    const int64_t per_row = p.N / 8;
    if (chunk >= (int64_t)p.R * per_row)
        return;
    const int64_t r = chunk / per_row;
    const int64_t col = (chunk - r * per_row) * 8;
    const int64_t row = (int64_t)mr.x * p.R + r;
    if (row >= p.m)
        return;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < mr.z; ++t) {
        const float *src = p.partial + ((int64_t)(mr.y + t) * p.R + r) * p.N + col;
        f32x4_t a = *reinterpret_cast<const f32x4_t *>(src);
        f32x4_t b = *reinterpret_cast<const f32x4_t *>(src + 4);
        s[0] += a[0]; s[1] += a[1]; s[2] += a[2]; s[3] += a[3];
        s[4] += b[0]; s[5] += b[1]; s[6] += b[2]; s[7] += b[3];
    }
    store_row<8>(p.C, row * p.ldc + col, p.c_dtype, s);
}

template <int FMT, int R, int V, int AB>
static hipError_t launch_one(const TileParams &p, dim3 grid, dim3 block, size_t lds,
                             hipStream_t stream)
{
    hipLaunchKernelGGL((spmm_tile_kernel<FMT, R, V, AB>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <int FMT, int R, int V>
static hipError_t by_ab(int ab, const TileParams &p, dim3 g, dim3 b, size_t lds, hipStream_t s)
{
    return ab == SPMM_FP16 ? launch_one<FMT, R, V, SPMM_FP16>(p, g, b, lds, s)
                           : launch_one<FMT, R, V, SPMM_BF16>(p, g, b, lds, s);
}

template <int FMT, int R>
static hipError_t by_v(int v, int ab, const TileParams &p, dim3 g, dim3 b, size_t lds,
                       hipStream_t s)
{
    switch (v) {
    case 2: return by_ab<FMT, R, 2>(ab, p, g, b, lds, s);
    case 4: return by_ab<FMT, R, 4>(ab, p, g, b, lds, s);
    default: return by_ab<FMT, R, 8>(ab, p, g, b, lds, s);
    }
}

template <int FMT>
static hipError_t by_r(int r, int v, int ab, const TileParams &p, dim3 g, dim3 b, size_t lds,
                       hipStream_t s)
{
    switch (r) {
    case 16: return by_v<FMT, 16>(v, ab, p, g, b, lds, s);
    case 32: return by_v<FMT, 32>(v, ab, p, g, b, lds, s);
    default: return by_v<FMT, 64>(v, ab, p, g, b, lds, s);
    }
}

size_t tile_lds_bytes(int R, int V, int waves_n, int waves_k)
{
    return waves_k > 1 ? (size_t)waves_n * (R / 16) * V * 4 * 64 * sizeof(float) : 0;
}

hipError_t launch_tiles(int fmt, int R, int V, int ab, const TileParams &p, int64_t n_items,
                        int64_t n_col_tiles, hipStream_t stream)
{
    dim3 grid((unsigned)n_items, (unsigned)n_col_tiles);
    dim3 block(64 * p.waves_n * p.waves_k);
    size_t lds = tile_lds_bytes(R, V, p.waves_n, p.waves_k);
    return fmt == 0 ? by_r<0>(R, V, ab, p, grid, block, lds, stream)
                    : by_r<1>(R, V, ab, p, grid, block, lds, stream);
}

hipError_t launch_merge(const MergeParams &p, int64_t n_merges, hipStream_t stream)
{
    const int64_t chunks = (int64_t)p.R * (p.N / 8);
    dim3 grid((unsigned)n_merges, (unsigned)((chunks + 255) / 256));
    hipLaunchKernelGGL(wcsr_merge_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace wspmm

// Device helpers shared by the gfx950 SpMM kernels: vector types, buffer
// resources and loads, the MFMA wrapper, output conversions and stores, the
// work-group numbering and an LDS-only barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "window_spmm.h"

namespace wspmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-class devices (no format conversion,
// no swizzle): the value the ROCm libraries use for gfx90a/gfx94x/gfx950.
constexpr int kRsrcWord3 = 0x00020000;
// Offset used for "no data": beyond any resource size the host allows.
constexpr uint32_t kOOB = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// Cache-policy bits of buffer instructions: non-temporal.  (Measured: on the
// generic kernel's A stream this is slower, the data then bypasses the MALL.)
constexpr int kNT = 2;

template <int DW, int POL = 0>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *out)
{
    if constexpr (DW == 4) {
        u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (DW == 2) {
        u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POL);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POL);
    }
}

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

// fp8 (OCP E4M3) MFMA: 8 codes of A and of B per lane, k = 8g .. 8g+7 for lane
// 16g + i, byte 0 first.
__device__ __forceinline__ f32x4_t mfma16x16x32_fp8(u32x2_t a, u32x2_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                      __builtin_bit_cast(long, b), c, 0, 0, 0);
}

// Byte transpose of one lane's 8 x 8 block: row j is b[j] (bytes 0-3 in b[j][0],
// 4-7 in b[j][1]); out[c] receives byte column c, rows 0-3 then rows 4-7 -- the
// MFMA B operand of column c.  Two rounds of byte selects: row pairs first
// ([r_j c, r_j+1 c] for two columns per word), then pairs of pairs.
__device__ __forceinline__ void transpose8x8_bytes(const uint32_t (&b)[8][2], u32x2_t (&out)[8])
{
    uint32_t ev[4][2], od[4][2];  // row pair, half hf: columns 4hf, 4hf+2 / 4hf+1, 4hf+3
#pragma unroll
    for (int pr = 0; pr < 4; ++pr)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            ev[pr][hf] = __builtin_amdgcn_perm(b[2 * pr + 1][hf], b[2 * pr][hf], 0x06020400u);
            od[pr][hf] = __builtin_amdgcn_perm(b[2 * pr + 1][hf], b[2 * pr][hf], 0x07030501u);
        }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < 2; ++w) {  // w = 0: rows 0-3 (pairs 0, 1); w = 1: rows 4-7
            out[4 * hf + 0][w] = __builtin_amdgcn_perm(ev[2 * w + 1][hf], ev[2 * w][hf], 0x05040100u);
            out[4 * hf + 2][w] = __builtin_amdgcn_perm(ev[2 * w + 1][hf], ev[2 * w][hf], 0x07060302u);
            out[4 * hf + 1][w] = __builtin_amdgcn_perm(od[2 * w + 1][hf], od[2 * w][hf], 0x05040100u);
            out[4 * hf + 3][w] = __builtin_amdgcn_perm(od[2 * w + 1][hf], od[2 * w][hf], 0x07060302u);
        }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Two fp32 results -> one word holding their 16-bit codes of type dt (low half
// first), rounded to nearest even by the hardware conversions (gfx950 converts
// a bfloat16 pair in one instruction; a NaN stays a NaN).
__device__ __forceinline__ uint32_t pack2(int dt, float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    if (dt == SPMM_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

// Stores V consecutive results of one row as c_dtype (NT: non-temporal stores).
template <typename T>
__device__ __forceinline__ void st(T *d, T x, bool nt)
{
    if (nt)
        __builtin_nontemporal_store(x, d);
    else
        *d = x;
}

template <int V, bool NT = false>
__device__ __forceinline__ void store_row(void *base, int64_t elem, int c_dtype, const float *v)
{
    if (c_dtype == SPMM_FP32) {
        float *d = reinterpret_cast<float *>(base) + elem;
        if constexpr (V >= 4) {
#pragma unroll
            for (int c = 0; c < V; c += 4)
                st(reinterpret_cast<f32x4_t *>(d + c), f32x4_t{v[c], v[c + 1], v[c + 2], v[c + 3]}, NT);
        } else {
            st(reinterpret_cast<f32x2_t *>(d), f32x2_t{v[0], v[1]}, NT);
        }
    } else {
        uint32_t w[V / 2];
#pragma unroll
        for (int c = 0; c < V; c += 2)
            w[c / 2] = pack2(c_dtype, v[c], v[c + 1]);
        uint16_t *d = reinterpret_cast<uint16_t *>(base) + elem;
        if constexpr (V == 8)
            st(reinterpret_cast<u32x4_t *>(d), u32x4_t{w[0], w[1], w[2], w[3]}, NT);
        else if constexpr (V == 4)
            st(reinterpret_cast<u32x2_t *>(d), u32x2_t{w[0], w[1]}, NT);
        else
            st(reinterpret_cast<uint32_t *>(d), w[0], NT);
    }
}

// Work-group id -> (work item, column tile), XCD-contiguous and column-tile major.
__device__ __forceinline__ void tile_of(int64_t n_items, int64_t total, int order, int64_t &item,
                                        int64_t &ctile)
{
    const int64_t i = blockIdx.x;
    const int64_t q = total >> 3, rem = total & 7;
    const int64_t xcd = i & 7, local = i >> 3;
    const int64_t logical = order ? i : xcd * q + (xcd < rem ? xcd : rem) + local;
    // (readfirstlane: tell the compiler these are wave-uniform, so that the
    // loads they address become scalar loads)
    ctile = __builtin_amdgcn_readfirstlane((int)(logical / n_items));
    item = __builtin_amdgcn_readfirstlane((int)(logical - ctile * n_items));
}

// Waits until this wave's LDS operations are done, then joins the work-group
// barrier.  Unlike __syncthreads() it does not wait for outstanding global
// loads, so prefetched B rows stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
    __builtin_amdgcn_s_barrier();
}

// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding: expcnt and lgkmcnt at
// their maxima, vmcnt split over bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// One pipeline stage of B: 8 gathered rows x DW dwords per lane.
template <int DW>
struct BStage {
    uint32_t b[8][DW];
};

}  // namespace wspmm

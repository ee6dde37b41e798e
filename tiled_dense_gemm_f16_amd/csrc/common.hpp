// Shared device-side pieces of the gfx950 GEMM + ReLU kernels: vector types,
// buffer descriptors, the launch-index -> tile mapping and the epilogue
// conversion.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "gemm_relu.h"

namespace gemm_relu {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((vector_size(8)));
typedef short i16x8 __attribute__((vector_size(16)));

#define GR_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
// An offset that is never inside a buffer: every descriptor is given at most
// this many bytes, so a lane loading here reads zeros (the edge masking).
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint64_t kMaxRecords = 0x80000000ull;
// Raw-buffer descriptor word 3 for gfx9 (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

struct Args {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;
    int order;  // GEMM_RELU_ORDER_*
    // split-K kernel only
    float* partial;      // [splits][M][N] fp32 partial sums (splits > 1)
    uint32_t* counters;  // one per column tile, zero between launches (splits > 1)
    int splits;          // workgroups along K
    int kc;              // K range of one workgroup
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes >= kMaxRecords ? (uint32_t)kMaxRecords : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Maps the launch index to a (tile_m, tile_n) pair.
//  1. XCD remap: workgroup b is dispatched to die b % 8 (each of the 8 dies
//     has its own L2). Renumber so that die x receives one contiguous range
//     of tile ids (a bijection for any count).
//  2. Grouped order: ids run down `group_m` tile-rows before moving to the next
//     tile-column, so tiles that run together on a die share A row-panels and
//     B column-panels in its L2 (the block-order swizzle of the TileLang GEMM
//     example).
__device__ __forceinline__ void tile_coords(const Args& a, int& tm, int& tn)
{
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if (a.order == GEMM_RELU_ORDER_ROW_MAJOR) {
        tm = bid / a.tiles_n;
        tn = bid % a.tiles_n;
        return;
    }
    {
        const int q = nblk / 8, r = nblk % 8;
        const int xcd = bid % 8, idx = bid / 8;
        bid = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    }
    const int gsize = a.group_m * a.tiles_n;
    const int g = bid / gsize;
    const int first_m = g * a.group_m;
    const int gm = min(a.tiles_m - first_m, a.group_m);
    const int in_g = bid - g * gsize;
    tm = first_m + in_g % gm;
    tn = in_g / gm;
}

// Transpose an 8x8 block of halves held as 8 rows of 16 bytes: out[c] holds
// column c (8 values, one per input row).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8])
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // low half from row 2j, high half from row 2j+1, both at column c
            out[c][j] = __builtin_amdgcn_perm(in[2 * j + 1][c >> 1], in[2 * j][c >> 1], sel);
        }
    }
}

// ReLU on an fp32 accumulator and the conversion to fp16, round to nearest
// even (v_cvt_f16_f32 under the default rounding mode), as a bit pattern.
__device__ __forceinline__ uint32_t relu_pack2(float lo, float hi)
{
    const _Float16 a = (_Float16)fmaxf(lo, 0.0f);
    const _Float16 b = (_Float16)fmaxf(hi, 0.0f);
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ uint16_t relu_f16(float x)
{
    return __builtin_bit_cast(uint16_t, (_Float16)fmaxf(x, 0.0f));
}

}  // namespace gemm_relu

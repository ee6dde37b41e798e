// Shared device-side pieces of the gfx950 GEMM + ReLU kernels: vector types,
// buffer descriptors, the launch-index -> tile mapping and the epilogue
// conversion.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "gemm_relu.h"

namespace gemm_relu {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    // operand layouts: 0 = as stored (A: M x K, B: K x N), 1 = the stored
    // matrix is the transpose (A: K x M, leading dim M; B: N x K, leading dim K)
    int trans_a, trans_b;
    // epilogue: kActRelu, or kActBiasGelu with bias[N] (fp16, one per column)
    int act;
    const uint16_t* bias;
    // split-K kernel only
    float* partial;      // [splits][M][N] fp32 partial sums (splits > 1)
    uint32_t* counters;  // one per column tile, zero between launches (splits > 1)
    int splits;          // workgroups along K
    int kc;              // K range of one workgroup
    // timestamp builds only (GR_STAMPS): kStampWords words per workgroup, or null
    uint64_t* stamps;
};

// Per-workgroup timestamps, compiled in only when GR_STAMPS is defined (the
// profiling build of build.py --stamps): the first wave keeps the 100 MHz
// realtime counter of a few points of a kernel in registers (constant slots,
// no memory traffic inside the kernel), and at the end its first lane writes
// them, with the die (XCC_ID) and hardware ids, to p.stamps. Slots: 0 start,
// 1 first tile data in LDS or registers, 2 main loop done, 3 last store
// acknowledged; 4 split-K partials stored and counted; 5 die, 6 HW_ID.
// Ordinary builds compile none of it.
constexpr int kStampWords = 8;
#ifdef GR_STAMPS
#define GR_STAMP_DECL uint64_t gr_stamps[kStampWords] = {}
#define GR_STAMP(i)                                          \
    do {                                                     \
        gr_stamps[i] = __builtin_amdgcn_s_memrealtime();     \
    } while (0)
#define GR_STAMP_FLUSH(p)                                                                   \
    do {                                                                                    \
        __builtin_amdgcn_s_waitcnt(0);                                                      \
        gr_stamps[3] = __builtin_amdgcn_s_memrealtime();                                    \
        if (threadIdx.x == 0 && (p).stamps) {                                               \
            unsigned gr_xcc, gr_hw;                                                         \
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(gr_xcc));            \
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(gr_hw));              \
            gr_stamps[5] = gr_xcc;                                                          \
            gr_stamps[6] = gr_hw;                                                           \
            _Pragma("unroll") for (int gr_k = 0; gr_k < kStampWords; ++gr_k)               \
                (p).stamps[(int64_t)blockIdx.x * kStampWords + gr_k] = gr_stamps[gr_k];     \
        }                                                                                   \
    } while (0)
#else
#define GR_STAMP_DECL static_assert(true, "")
#define GR_STAMP(i) \
    do {            \
    } while (0)
#define GR_STAMP_FLUSH(p) \
    do {                  \
    } while (0)
#endif

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

// Epilogues. ReLU is the GEMM + ReLU example's ("Writing high-performance
// kernels in TileLang", section "Escribamos un GEMM"); bias + GELU is the
// fused epilogue of "TileLang simplifica la creación de kernels GPU de alto
// rendimiento" (section "Fusionar operaciones para reducir viajes a
// memoria"): v + bias[n], then GELU(x) = x * Phi(x), Phi the standard normal
// distribution function, all in fp32.
constexpr int kActRelu = 0;
constexpr int kActBiasGelu = 1;

__device__ __forceinline__ float relu(float x) { return fmaxf(x, 0.0f); }

// erfc(z) for z >= 0 with a fractional error below 1.2e-7 at every z: the
// Chebyshev-fitted approximation of Numerical Recipes (Press, Teukolsky,
// Vetterling, Flannery; section 6.2, "erfcc"),
//   erfc(z) ~ t * exp(-z^2 + P(t)),  t = 1 / (1 + z/2),
// P a degree-9 polynomial, evaluated here by Horner's rule: one reciprocal,
// nine FMAs and one exp, against about fifty instructions for the library's
// erfcf. In fp32 the result stays within a few parts in 1e6 of erfc, far
// below the fp16 output's resolution.
__device__ __forceinline__ float erfc_nonneg(float z)
{
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    float s = 0.17087277f;
    s = fmaf(s, t, -0.82215223f);
    s = fmaf(s, t, 1.48851587f);
    s = fmaf(s, t, -1.13520398f);
    s = fmaf(s, t, 0.27886807f);
    s = fmaf(s, t, -0.18628806f);
    s = fmaf(s, t, 0.09678418f);
    s = fmaf(s, t, 0.37409196f);
    s = fmaf(s, t, 1.00002368f);
    s = fmaf(s, t, -1.26551223f);
    return t * __expf(fmaf(-z, z, s));
}

// GELU(x) = x * Phi(x). With q = Phi(-|x|) = erfc(|x| / sqrt 2) / 2 (always in
// (0, 1/2], no cancellation): x * q for x < 0, x - x * q for x >= 0.
__device__ __forceinline__ float gelu(float x)
{
    const float q = 0.5f * erfc_nonneg(fabsf(x) * 0.70710678118654752f);
    return x < 0.0f ? x * q : fmaf(-x, q, x);
}

// bias of column n (zero past N, where nothing is stored)
__device__ __forceinline__ float bias_at(const Args& p, int n)
{
    return n < p.N ? (float)__builtin_bit_cast(_Float16, p.bias[n]) : 0.0f;
}

// Two fp32 values to a packed pair of fp16, each rounded to nearest even
// (v_cvt_pk_f16_f32 under the default rounding mode; never the
// round-toward-zero pack).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// ReLU of a pair, applied after the rounding: max(fp16(x), 0) is fp16(max(x,
// 0)) for every x (a positive x rounds to a value >= +0, a negative one to a
// value <= 0 that the max turns into +0, and a sum that is exactly zero is
// +0), and costs one packed conversion and one packed max per pair instead
// of two maxima, two conversions and a merge.
__device__ __forceinline__ uint32_t relu_pack_f16x2(float lo, float hi)
{
    const f16x2 h = __builtin_convertvector(f32x2{lo, hi}, f16x2);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(h, f16x2{(_Float16)0.0f, (_Float16)0.0f}));
}

// Bias of columns n .. n+3 (n % 4 == 0, N % 8 == 0: the vector paths), one
// 8-byte load; columns past N read zeros.
__device__ __forceinline__ f32x4 bias4(const Args& p, int n)
{
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p.bias, (uint64_t)p.N * 2);
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, n < p.N ? n * 2 : (int)kOOB, 0, 0);
    f32x4 b;
    b[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xFFFF));
    b[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16));
    b[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] & 0xFFFF));
    b[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] >> 16));
    return b;
}

// Two consecutive outputs with their biases already loaded.
template <int ACT>
__device__ __forceinline__ uint32_t epi_pack2b(float lo, float hi, float blo, float bhi)
{
    if constexpr (ACT == kActBiasGelu) return pack_f16x2(gelu(lo + blo), gelu(hi + bhi));
    else return relu_pack_f16x2(lo, hi);
}

template <int ACT>
__device__ __forceinline__ uint16_t epi_f16(const Args& p, float x, int n)
{
    const float y = (ACT == kActBiasGelu) ? gelu(x + bias_at(p, n)) : relu(x);
    return __builtin_bit_cast(uint16_t, (_Float16)y);
}

// Runs body.template operator()<ACT>() with the epilogue the call asked for:
// one branch around the whole epilogue, none in the main loop.
template <class F>
__device__ __forceinline__ void with_epilogue(const Args& p, F&& body)
{
    if (p.act == kActBiasGelu) body.template operator()<kActBiasGelu>();
    else body.template operator()<kActRelu>();
}

}  // namespace gemm_relu

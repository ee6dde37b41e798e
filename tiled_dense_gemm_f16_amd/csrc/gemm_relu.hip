// C = ReLU(A @ B) for fp16 A[M,K], B[K,N] on MI355X (gfx950, CDNA4): the
// host side of the C ABI declared in include/gemm_relu.h.
//
// The computation is the GEMM + ReLU example of "Writing high-performance
// kernels in TileLang" (section "Escribamos un GEMM"). Three kernel families
// implement it:
//  * pipelined.hpp -- the large-tile hot path: direct-to-LDS loads, a
//    four-stage LDS ring, v_mfma_f32_32x32x16_f16, transposing LDS reads;
//  * staged.hpp    -- register-staged loads with v_mfma_f32_16x16x32_f16, for
//    small tiles and for the generic element-wise path (any K, N, alignment);
//  * splitk.hpp    -- few rows: B streamed through registers, K split across
//    waves and workgroups, fp32 partials combined by the last workgroup.
// This file holds the tile table, the shape heuristic, argument validation,
// the split-K workspaces and the launches.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "gemm_relu.h"
#include "pipelined.hpp"
#include "small.hpp"
#include "splitk.hpp"
#include "staged.hpp"

namespace {

// ---------------------------------------------------------------------------
// Tile table
// ---------------------------------------------------------------------------

using gemm_relu::Args;

using P256 = gemm_relu::pipelined::Cfg<256, 256, 2, 2>;   // 4 waves x 128x128, 32x32x16 MFMA
using P256W8 = gemm_relu::pipelined::Cfg<256, 256, 4, 2>; // 8 waves x 64x128: two waves per SIMD
using P256S5 = gemm_relu::pipelined::Cfg<256, 256, 2, 2, 5>; // five-slot ring: 4 steps in flight
using P128 = gemm_relu::pipelined::Cfg<128, 256, 2, 2>;      // 4 waves x 64x128
using P64 = gemm_relu::pipelined::Cfg<64, 256, 1, 2>;        // 2 waves x 64x128
// The same with a five-slot ring (4 steps in flight, 100 KiB: one workgroup
// per CU). On grids of at most one workgroup per CU it is 5-12 % faster
// (2048^3 31.7 -> 30.0 us, 4096 x 1024 x 4096 57.4 -> 52.2, TN 256 x 8192 x
// 8192 107.8 -> 94.3); on larger grids two four-slot workgroups share a CU
// and the deeper ring loses (2560^3 with this tile: 48.6 -> 68.1 us).
using P64S5 = gemm_relu::pipelined::Cfg<64, 256, 1, 2, 5>;
// 256 x 256 with A (stored M x K) loaded two steps at a time: whole 128-byte
// lines per row, 256 L2 requests per step and CU instead of 384
using P256AP = gemm_relu::pipelined::Cfg<256, 256, 2, 2, 4, true>;
using P128AP = gemm_relu::pipelined::Cfg<128, 256, 2, 2, 4, true>;  // the same for 128 x 256
using P64AP = gemm_relu::pipelined::Cfg<64, 256, 1, 2, 4, true>;    // and 64 x 256
using Q64 = gemm_relu::small::Cfg<64, 64, 2, 2, 2, 4>;     // 4 waves x 32x32, 64-deep steps, 4 slots
using Q32 = gemm_relu::small::Cfg<32, 64, 1, 2, 2, 4>;     // 2 waves x 32x32, 64-deep steps, 4 slots
using S256 = gemm_relu::staged::Tile<256, 256, 64, 2, 2>;  // generic instance of the same tile
using S128 = gemm_relu::staged::Tile<128, 128, 64, 2, 2, 1, 3>;  // the pages' 128x128x64 tile
using S64 = gemm_relu::staged::Tile<64, 64, 64, 2, 2, 1, 4>;      // 4 waves x 32x32
using S16 = gemm_relu::staged::Tile<16, 64, 64, 1, 4, 1, 4>;      // 4 waves x 16x16: few rows
#ifndef GR_SPLITK_NW
#define GR_SPLITK_NW 4
#endif
// steps of 32 rows in flight per split-K wave: 2 measured 0.4-6 % faster than
// 4 on every split-K launch of the sweep (1000 x 1016 x 1000 11.55 -> 10.90
// us, 16 x 8192 x 8192 30.36 -> 30.24), 3 in between and 6 slower
#ifndef GR_SPLITK_D
#define GR_SPLITK_D 2
#endif
using K16 = gemm_relu::splitk::Cfg<1, GR_SPLITK_NW, GR_SPLITK_D>;  // split-K, 16 rows x 128 columns
using K32 = gemm_relu::splitk::Cfg<2, GR_SPLITK_NW, GR_SPLITK_D>;  // split-K, 32 rows x 128 columns
using K64 = gemm_relu::splitk::Cfg<4, GR_SPLITK_NW, GR_SPLITK_D>;  // split-K, 64 rows x 128 columns

using LaunchFn = hipError_t (*)(const Args&, hipStream_t);

// Each launcher instantiates its kernel for the four operand layouts
// (A as stored or transposed) x (B as stored or transposed).
template <class T, bool VEC, bool TA, bool TB>
void launch_staged_as(const Args& a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_relu::staged::staged_kernel<T, VEC, TA, TB>), dim3(a.tiles_m * a.tiles_n), dim3(T::NT),
                       0, s, a);
}

template <class T, bool VEC>
hipError_t launch_staged(const Args& a, hipStream_t s)
{
    switch (2 * a.trans_a + a.trans_b) {
    case 0: launch_staged_as<T, VEC, false, false>(a, s); break;
    case 1: launch_staged_as<T, VEC, false, true>(a, s); break;
    case 2: launch_staged_as<T, VEC, true, false>(a, s); break;
    default: launch_staged_as<T, VEC, true, true>(a, s); break;
    }
    return hipGetLastError();
}

template <class T, bool TA, bool TB>
void launch_pipelined_as(const Args& a, hipStream_t s)
{
    const int blocks = a.tiles_m * a.tiles_n;
    if (a.K % T::BK == 0)
        hipLaunchKernelGGL((gemm_relu::pipelined::pipelined_kernel<T, true, TA, TB>), dim3(blocks), dim3(T::NT), 0,
                           s, a);
    else
        hipLaunchKernelGGL((gemm_relu::pipelined::pipelined_kernel<T, false, TA, TB>), dim3(blocks), dim3(T::NT), 0,
                           s, a);
}

template <class T>
hipError_t launch_pipelined(const Args& a, hipStream_t s)
{
    switch (2 * a.trans_a + a.trans_b) {
    case 0: launch_pipelined_as<T, false, false>(a, s); break;
    case 1: launch_pipelined_as<T, false, true>(a, s); break;
    case 2: launch_pipelined_as<T, true, false>(a, s); break;
    default: launch_pipelined_as<T, true, true>(a, s); break;
    }
    return hipGetLastError();
}

// The small-tile kernel covers operands as stored (NN); with a transposed
// operand the register-staged kernel of the same tile size runs instead.
template <class T, class Fallback>
hipError_t launch_small(const Args& a, hipStream_t s)
{
    if (a.trans_a || a.trans_b) return launch_staged<Fallback, true>(a, s);
    const int blocks = a.tiles_m * a.tiles_n;
    if (a.K % T::BK == 0)
        hipLaunchKernelGGL((gemm_relu::small::small_kernel<T, true>), dim3(blocks), dim3(T::NT), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_relu::small::small_kernel<T, false>), dim3(blocks), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

template <class T, bool TA, bool TB>
void launch_splitk_as(const Args& a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_relu::splitk::splitk_kernel<T, TA, TB>), dim3(a.tiles_m * a.tiles_n * a.splits),
                       dim3(T::NT), 0, s, a);
}

template <class T>
hipError_t launch_splitk(const Args& a, hipStream_t s)
{
    switch (2 * a.trans_a + a.trans_b) {
    case 0: launch_splitk_as<T, false, false>(a, s); break;
    case 1: launch_splitk_as<T, false, true>(a, s); break;
    case 2: launch_splitk_as<T, true, false>(a, s); break;
    default: launch_splitk_as<T, true, true>(a, s); break;
    }
    return hipGetLastError();
}

// Launch parameters of each family's configurations, for gemm_relu_tile_info.
template <class T>
constexpr gemm_relu_tile_desc pipelined_desc(int group_m)
{
    return {T::BM, T::BN, T::BK, T::STAGES, T::WAVES_M, T::WAVES_N, 1, T::NT, T::STAGES * T::STAGE_BYTES,
            0, group_m, GEMM_RELU_FAMILY_PIPELINED, {0, 0, 0, 0}};
}

template <class T>
constexpr gemm_relu_tile_desc small_desc(int group_m)
{
    return {T::BM, T::BN, T::BK, T::STAGES, T::WAVES_M, T::WAVES_N, 1, T::NT, T::STAGES * T::SLOT * 2,
            0, group_m, GEMM_RELU_FAMILY_SMALL, {0, 0, 0, 0}};
}

template <class T>
constexpr gemm_relu_tile_desc staged_desc(int group_m)
{
    return {T::BM, T::BN, T::BK, 2, T::WAVES_M, T::WAVES_N, 1, T::NT, T::LDS_BYTES,
            0, group_m, GEMM_RELU_FAMILY_STAGED, {0, 0, 0, 0}};
}

template <class T>
constexpr gemm_relu_tile_desc splitk_desc()
{
    return {T::BM, T::TN, T::BK, T::D, 1, 1, T::NW, T::NT,
            (int)(sizeof(float) * T::NW * T::BM * T::RED_ROW + sizeof(uint32_t)),
            1, 1, GEMM_RELU_FAMILY_SPLITK, {0, 0, 0, 0}};
}

struct TileEntry {
    const char* name;
    gemm_relu_tile_desc desc;
    LaunchFn vec;     // K % 8 == 0, N % 8 == 0, 16-byte aligned pointers
    LaunchFn generic; // anything else
};

const TileEntry kTiles[] = {
    {"256x256x32s4_w2x2_mfma32x32x16_lds-dma", pipelined_desc<P256>(4), launch_pipelined<P256>,
     launch_staged<S256, false>},
    {"128x128x64_w2x2_mfma16x16x32", staged_desc<S128>(4), launch_staged<S128, true>,
     launch_staged<S128, false>},
    {"64x64x64_w2x2_mfma16x16x32", staged_desc<S64>(4), launch_staged<S64, true>, launch_staged<S64, false>},
    {"16x64x64_w1x4_mfma16x16x32", staged_desc<S16>(1), launch_staged<S16, true>, launch_staged<S16, false>},
    {"splitk_16x128_w4k_mfma16x16x32_regT", splitk_desc<K16>(), launch_splitk<K16>, launch_staged<S16, false>},
    {"splitk_32x128_w4k_mfma16x16x32_regT", splitk_desc<K32>(), launch_splitk<K32>, launch_staged<S64, false>},
    {"splitk_64x128_w4k_mfma16x16x32_regT", splitk_desc<K64>(), launch_splitk<K64>, launch_staged<S64, false>},
    {"256x256x32s4_w4x2_mfma32x32x16_lds-dma", pipelined_desc<P256W8>(4), launch_pipelined<P256W8>,
     launch_staged<S256, false>},
    {"256x256x32s5_w2x2_mfma32x32x16_lds-dma", pipelined_desc<P256S5>(4), launch_pipelined<P256S5>,
     launch_staged<S256, false>},
    {"128x256x32s4_w2x2_mfma32x32x16_lds-dma", pipelined_desc<P128>(4), launch_pipelined<P128>,
     launch_staged<S128, false>},
    {"64x256x32s4_w1x2_mfma32x32x16_lds-dma", pipelined_desc<P64>(4), launch_pipelined<P64>,
     launch_staged<S64, false>},
    {"64x64x64s4_w2x2_mfma32x32x16_lds-small", small_desc<Q64>(8), launch_small<Q64, S64>,
     launch_staged<S64, false>},
    {"32x64x64s4_w1x2_mfma32x32x16_lds-small", small_desc<Q32>(4), launch_small<Q32, S64>,
     launch_staged<S64, false>},
    {"64x256x32s5_w1x2_mfma32x32x16_lds-dma", pipelined_desc<P64S5>(4), launch_pipelined<P64S5>,
     launch_staged<S64, false>},
    {"256x256x32s4_w2x2_mfma32x32x16_lds-dma-a2", pipelined_desc<P256AP>(4), launch_pipelined<P256AP>,
     launch_staged<S256, false>},
    {"128x256x32s4_w2x2_mfma32x32x16_lds-dma-a2", pipelined_desc<P128AP>(4), launch_pipelined<P128AP>,
     launch_staged<S128, false>},
    {"64x256x32s4_w1x2_mfma32x32x16_lds-dma-a2", pipelined_desc<P64AP>(4), launch_pipelined<P64AP>,
     launch_staged<S64, false>},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kP64Tile = 10, kP64S5Tile = 13;  // 64 x 256 with four and with five slots
// the same tiles with A (stored M x K) loaded two steps at a time
constexpr int kP256Tile = 0, kP256PairTile = 14;
constexpr int kP128Tile = 9, kP128PairTile = 15;
constexpr int kP64PairTile = 16;

// The group a launch without opts uses: the tile's default, cut to a power of
// two that leaves at least two groups when the grid has four tile-rows or
// more. A group spanning every tile-row measured 3-5 % slower on average over
// the sweeps than 4 or 8 rows (384 x 6144 x 6144 with 64 x 64 tiles, 6 rows:
// 84.9 us in one group of 6 against 77.6 in groups of 4).
int default_group(int group, int tiles_m)
{
    int g = 1;
    while (2 * g <= group && 2 * g <= tiles_m) g *= 2;
    if (g == tiles_m && tiles_m >= 4) g /= 2;
    return g;
}
constexpr int kGenericTile = 2;  // tile used by the element-wise path
constexpr int kSplitKTN = 128;   // columns of a split-K workgroup
constexpr int kSplitKStep = GR_SPLITK_NW * 32;  // K granularity of a split-K workgroup (waves x 32)

// How many workgroups share the K range of one split-K tile, and the K range
// of each (a multiple of kSplitKStep). Candidates are powers of two up to one
// step per workgroup and at most one workgroup per CU (a second round never
// paid in the sweeps); among them the one with the least predicted time:
//   a fixed part + a cost per split (partials written, counted and re-read
//   by the last workgroup) + the streaming of B, bytes over the smaller of
//   (workgroups x one CU's streaming rate) and the HBM rate + the serial depth
//   of one workgroup's K range.
// The constants were fitted to split-K launches of 16 x N x K (N = 1024 to
// 8192, K = 2048 to 8192) with 1 to 64 splits; for those shapes the model's
// choice is the measured best or within 4 % of it.
constexpr double kSplitPerSplitUs = 0.431;
constexpr double kSplitCuBytesPerUs = 58.07e3;   // one CU streaming B
constexpr double kSplitHbmBytesPerUs = 6.18e6;   // all CUs streaming B
constexpr double kSplitDepthUsPer1024 = 1.89;    // per 1024 rows of a workgroup's K range
constexpr int64_t kSplitMaxWorkgroups = 256;     // one per CU
constexpr int64_t kMaxSplitPartialBytes = (int64_t)1 << 31;  // one split's M x N fp32 partials

void choose_splits(int64_t M, int64_t N, int64_t K, int64_t tiles, int& splits, int& kc)
{
    const int64_t max_s = (K + kSplitKStep - 1) / kSplitKStep;  // at least one step per workgroup
    const double bytes = (double)tiles * kSplitKTN * (double)K * 2.0;  // B, once per row tile
    double best = 0.0;
    splits = 1;
    kc = (int)((K + kSplitKStep - 1) / kSplitKStep * kSplitKStep);
    if (kc < kSplitKStep) kc = kSplitKStep;
    // the combine reads one split's M x N fp32 partials through a buffer
    // descriptor, whose range ends below 2^31 bytes
    if (M * N * 4 >= kMaxSplitPartialBytes) return;
    for (int64_t s = 1; s <= max_s; s *= 2) {
        int64_t c = (K + s - 1) / s;
        c = (c + kSplitKStep - 1) / kSplitKStep * kSplitKStep;
        if (c < kSplitKStep) c = kSplitKStep;
        const int64_t se = (K + c - 1) / c < 1 ? 1 : (K + c - 1) / c;
        const int64_t wgs = tiles * se;
        if (se > 1 && wgs > kSplitMaxWorkgroups) break;
        const double rate = (double)wgs * kSplitCuBytesPerUs < kSplitHbmBytesPerUs
                                ? (double)wgs * kSplitCuBytesPerUs : kSplitHbmBytesPerUs;
        const double us = kSplitPerSplitUs * (double)se + bytes / rate + kSplitDepthUsPer1024 * (double)c / 1024.0;
        if (s == 1 || us < best) {
            best = us;
            splits = (int)se;
            kc = (int)c;
        }
    }
}

// The vector kernels: 16-byte aligned pointers and leading dimensions (K or M
// for A, N or K for B, N for C) that are multiples of 8 halves.
bool fast_path_ok(int64_t M, int64_t N, int64_t K, bool ta, bool tb, const void* A, const void* B, const void* C)
{
    const uintptr_t mis = ((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15u;
    const int64_t lda = ta ? M : K, ldb = tb ? K : N;
    // 32-bit in-tile buffer offsets: 256 rows of K halves, 64 rows of M or N
    // halves, stay below 2^31 bytes
    return lda % 8 == 0 && ldb % 8 == 0 && N % 8 == 0 && mis == 0 && K <= (1 << 22) && N <= (1 << 24) &&
           (!ta || M <= (1 << 24));
}

// The split-K kernel addresses A with 32-bit offsets.
bool splitk_ok(int64_t M, int64_t K) { return M * K * 2 < ((int64_t)1 << 31); }

// The shape heuristic: a cost model whose constants were fitted to offline
// sweeps (tune.py) of every tile and block order: 38 shapes in the NN layout,
// from 1 to 8192 rows, 64 to 8192 columns and 256 to 12288 deep, and 12 shapes
// in each transposed layout. A tile's predicted time is
//   rounds x (2 bm bn kc FLOP) / rate,   rounds = ceil(workgroups / 256),
// floored by the HBM time of the algorithmic bytes, plus for split-K launches
// the cost of writing and re-reading the fp32 partials and of the combine.
// The rate is what one compute unit sustains on that tile in that operand
// layout (larger tiles reuse each loaded byte more; the fitted rates include
// the clock the chip holds under load). Two rules sit on top: few rows
// (M <= 32 with operands as stored, M <= 64 otherwise) always take a split-K
// tile, and the 16x64 tile is only for latency-bound outputs of at most 64 K
// elements. Over the offline sweeps the default launch (this model, the
// small-tile model below, the group and block-order rules) is 2.3-2.7 %
// slower than the measured fastest on average in NN over two sweeps (12-17 %
// at worst; 46 shapes) and 1.2-3.0 % in the transposed layouts (12 shapes
// each; 11-18 % at worst, TT 4096 x 64 x 4096, where the split-K tile is
// chosen over the 64 x 256 one).
// The rules it
// replaced, which looked at M and the 256x256 tile count alone, were up to
// 6x slower on shapes they were not written for.
struct AutoTile {
    int id;
    double tflops_per_cu[4];  // NN, NT, TN, TT (index 2 * trans_a + trans_b)
};
constexpr AutoTile kAutoTiles[] = {
    {0, {6.96, 5.78, 6.63, 6.10}},   // 256x256 pipelined
    {9, {5.24, 3.90, 4.96, 4.04}},   // 128x256 pipelined
    // 64x256 pipelined (TN: refit after the step-descriptor change; NT: refit
    // when it came to load A two steps at a time)
    {10, {3.21, 2.43, 3.49, 2.25}},
    {6, {2.13, 1.15, 0.570, 0.517}}, // split-K 64x128
    {5, {1.48, 0.772, 0.390, 0.344}},// split-K 32x128
    {4, {1.12, 0.472, 0.408, 0.324}},// split-K 16x128
    {2, {0.895, 1.24, 0.429, 0.756}},// 64x64 staged
    // 128x128 staged: with B stored N x K (NT) it needs no transpose and beat
    // the pipelined tiles at 2048^3 and 4096 x 1024 x 4096 (39.1 against
    // 40.7 us, 71.1 against 76.8) until the 64 x 256 tile came to load A two
    // steps at a time (34.4-37.9 against 39.7 us, 66.3 against 72.2); its
    // other rates keep it out of the NN, TN and TT choices, where it was
    // 1.15-3x off the best.
    {1, {1.0, 2.35, 0.9, 1.4}},
    {3, {0.273, 0.706, 0.118, 0.262}},// 16x64 staged
};
// The small tiles (direct-to-LDS, NN only) on the problems they fill: their
// time is a fixed part (first loads' latency, epilogue) plus the bytes each
// compute unit loads at the rate this access pattern sustains per unit
// (64 x 64 tiles: 4.7 us at 256^3, 9.1 us at 1024^3, 22.8 us at 1536^3). Rows
// of A or B that are not whole 128-byte lines take more L2 requests (1000 x
// 1016 x 1000: 13.6 us against 9.1 at 1024^3). The three constants were
// chosen on a sweep of 46 shapes (every tile and block order, inputs from
// HBM) for the choices they lead to against the other tiles' predictions.
// After the skewed K walks and the step-descriptor cursor made the small and
// pipelined kernels faster, a coordinate search over the constants on a new
// sweep of every layout (82 shapes) lowered the fixed part (2.25 -> 1.80 us),
// the NN rate of the 32 x 128 split-K tile (1.59 -> 1.48) and the TN rate of
// the 64 x 256 tile (2.79 -> 3.49): 4096 x 512 x 4096, 1024 x 64 x 8192 and
// TN 4096 x 64 x 4096 now take the tiles that were 10-14 % faster there.
struct SmallTile {
    int id;
    bool one_round;  // only for grids of at most one workgroup per CU
};
// The 32 x 64 tile moves 1.5x the bytes of the 64 x 64 one per FLOP; it pays
// only where the 64 x 64 grid leaves CUs idle and its own grid still fits one
// round: with a partial second round (768^3: 288 workgroups) the units that
// run two take twice as long (8.8 us against 7.2 for 64 x 64).
constexpr SmallTile kSmallTiles[] = {{11, false}, {12, true}};
constexpr double kSmallFixedUs = 1.80;
// The rate model below predicts times that are, over the sweep, about
// 1.455 x + 4.0 us short of the measured ones (4096^3: 77 -> 116 us, 2048^3:
// 20.9 -> 34.4 us, 1024^3 split-K: 5.3 -> 11.9 us); a small tile's time is
// mapped into the same units before the two are compared.
constexpr double kRateModelScale = 1.455;
constexpr double kRateModelOffsetUs = 4.0;
constexpr double kSmallBytesPerUsPerCu = 44.0e3;  // 44 GB/s
constexpr double kSmallMisalignedRows = 0.40;     // extra per operand whose rows are not whole lines

constexpr double kComputeUnits = 256.0;
constexpr double kHbmBytesPerUs = 6.68e6;          // 6.68 TB/s
constexpr double kStagedHbmShare = 0.75;           // the register-staged kernels reach less of it
constexpr double kPartialUsPerByte = 0.97e-6;      // partials: written once, read once
constexpr double kCombineUs = 3.25;                // last-workgroup combine and counters

struct Prediction {
    double us;       // predicted time
    double compute;  // its compute part: breaks ties between HBM-bound tiles
};

Prediction predict(const AutoTile& at, int layout, int64_t M, int64_t N, int64_t K)
{
    const gemm_relu_tile_desc& d = kTiles[at.id].desc;
    const int64_t tiles = ((M + d.bm - 1) / d.bm) * ((N + d.bn - 1) / d.bn);
    int splits = 1, kc = (int)K;
    if (d.split_k) choose_splits(M, N, K, tiles, splits, kc);
    const double rounds = (double)((tiles * splits + (int64_t)kComputeUnits - 1) / (int64_t)kComputeUnits);
    const double compute = rounds * 2.0 * d.bm * d.bn * (double)kc / (at.tflops_per_cu[layout] * 1e6);
    const double bw = kHbmBytesPerUs * (d.family == GEMM_RELU_FAMILY_STAGED ? kStagedHbmShare : 1.0);
    const double memory = 2.0 * ((double)M * K + (double)K * N + (double)M * N) / bw;
    const double combine = splits > 1 ? kPartialUsPerByte * 8.0 * (double)M * N * splits + kCombineUs : 0.0;
    return {(compute > memory ? compute : memory) + combine, compute};
}

// The block order of a launch whose opts leave it to the library. On a grid
// of one round (every tile resident at once) of tiles of fewer than 256 rows,
// with two tile-rows or more, a multiple of 4 tile-columns and at least half
// as many tile-columns as tile-rows, plain row-major order ran 3-5 % faster
// than the grouped one in two tile sweeps at 256^3, 512^3, 768^3 and 1024^3,
// and 1-2 % on the wide skinny shapes (deep-K squares such as 1024 x 1024 x
// 4096 land within +-5 % either way from run to run); the grouped order wins
// on taller grids, on grids of several rounds and with the 256 x 256 tiles.
int default_order(const gemm_relu_tile_desc& d, int64_t tiles_m, int64_t tiles_n)
{
    const bool one_round = tiles_m * tiles_n <= (int64_t)kComputeUnits;
    return (!d.split_k && d.bm < 256 && one_round && tiles_m >= 2 && tiles_n % 4 == 0 && tiles_m <= 2 * tiles_n)
               ? GEMM_RELU_ORDER_ROW_MAJOR
               : GEMM_RELU_ORDER_DEFAULT;
}

// Predicted time of a small tile (operands as stored).
double predict_small(const SmallTile& st, int64_t M, int64_t N, int64_t K)
{
    const gemm_relu_tile_desc& d = kTiles[st.id].desc;
    const double wgs = (double)(((M + d.bm - 1) / d.bm) * ((N + d.bn - 1) / d.bn));
    // bytes one compute unit loads: workgroups are handed out as units free
    // up, so a unit's share is the average (at least one workgroup)
    const double per_cu = wgs / kComputeUnits;
    const double bytes = (per_cu > 1.0 ? per_cu : 1.0) * (double)(d.bm + d.bn) * (double)K * 2.0;
    const double misaligned = 1.0 + ((K * 2) % 128 ? kSmallMisalignedRows : 0.0) + ((N * 2) % 128 ? kSmallMisalignedRows : 0.0);
    return kSmallFixedUs + bytes * misaligned / kSmallBytesPerUsPerCu;
}

// The tile of least predicted time; among tiles bound by the same HBM time,
// the one with the least compute (the fewest padded rows).
int choose_tile(int64_t M, int64_t N, int64_t K, bool ta, bool tb)
{
    const bool sk = splitk_ok(M, K);
    const int layout = 2 * (ta ? 1 : 0) + (tb ? 1 : 0);
    // few rows: only the split-K tiles (up to 64 rows with a transposed
    // operand; with operands as stored the 32 x 64 small tile competes from
    // 33 rows on)
    const bool few_rows = M <= (layout == 0 ? 32 : 64) && sk;
    int best = -1;
    Prediction bp{0.0, 0.0};
    for (const AutoTile& at : kAutoTiles) {
        const gemm_relu_tile_desc& d = kTiles[at.id].desc;
        if (d.split_k ? !sk : few_rows) continue;
        if (at.id == 3 && M * N > 65536) continue;
        const Prediction p = predict(at, layout, M, N, K);
        const bool tie = p.us - bp.us < 1e-9 * bp.us && bp.us - p.us < 1e-9 * bp.us;
        if (best < 0 || (tie ? p.compute < bp.compute : p.us < bp.us)) {
            best = at.id;
            bp = p;
        }
    }
    // the small tiles: operands as stored, more than a few rows
    if (layout == 0 && !few_rows) {
        for (const SmallTile& st : kSmallTiles) {
            const gemm_relu_tile_desc& d = kTiles[st.id].desc;
            if (st.one_round && ((M + d.bm - 1) / d.bm) * ((N + d.bn - 1) / d.bn) > (int64_t)kComputeUnits) continue;
            const double us = (predict_small(st, M, N, K) - kRateModelOffsetUs) / kRateModelScale;
            if (us < bp.us) {
                best = st.id;
                bp = {us, 0.0};
            }
        }
    }
    // The pipelined tiles with A stored M x K load it two steps at a time
    // (whole cache lines: 3-14 % faster at 256 x 256, 7-8 % at 128 x 256;
    // at 64 x 256, 9-13 % in NT and on a par with the five-slot ring in NN).
    // With A stored K x M, 64 x 256 on a grid of one round takes the
    // five-slot ring.
    if (!ta) {
        if (best == kP256Tile) best = kP256PairTile;
        else if (best == kP128Tile) best = kP128PairTile;
        else if (best == kP64Tile) best = kP64PairTile;
    } else if (best == kP64Tile && ((M + 63) / 64) * ((N + 255) / 256) <= (int64_t)kComputeUnits) {
        best = kP64S5Tile;
    }
    return best;
}

// ---------------------------------------------------------------------------
// Split-K workspaces: one per (device, stream), grown on demand. The first
// `counter_slots` 32-bit words are tile counters, zero between launches (each
// launch's last workgroup resets the counters it used); the fp32 partial sums
// follow at a 256-byte boundary.
// ---------------------------------------------------------------------------

struct Workspace {
    char* base = nullptr;
    size_t counter_slots = 0;
    size_t partial_bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Workspaces replaced by larger ones. They are never freed: a HIP graph
// captured on that stream earlier holds their addresses in its kernel
// arguments and may be replayed at any time. Growth at least doubles both
// parts, so the retired buffers of a stream add up to less than its current
// workspace.
std::vector<char*> g_ws_retired;

size_t counter_bytes(size_t slots) { return (slots * 4 + 255) / 256 * 256; }

int get_workspace(int dev, hipStream_t stream, size_t slots, size_t partial_bytes, uint32_t** counters,
                  float** partial)
{
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace& w = g_ws[std::make_pair(dev, stream)];
    if (w.base == nullptr || w.counter_slots < slots || w.partial_bytes < partial_bytes) {
        // creating or growing the workspace allocates, synchronises and clears
        // it with a memset on the stream: none of that may be recorded into a
        // graph, so a stream under capture must already have a workspace large
        // enough (one such call made on it outside capture)
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return GEMM_RELU_EHIP;
        if (cap != hipStreamCaptureStatusNone) return GEMM_RELU_EUNSUPPORTED;
        size_t ns = slots > w.counter_slots ? slots : w.counter_slots;
        size_t np = partial_bytes > w.partial_bytes ? partial_bytes : w.partial_bytes;
        if (w.base != nullptr) {
            ns = ns > 2 * w.counter_slots ? ns : 2 * w.counter_slots;
            np = np > 2 * w.partial_bytes ? np : 2 * w.partial_bytes;
        }
        char* p = nullptr;
        if (hipMalloc(reinterpret_cast<void**>(&p), counter_bytes(ns) + np) != hipSuccess) {
            (void)hipGetLastError();
            return GEMM_RELU_ENOMEM;
        }
        if (hipMemsetAsync(p, 0, counter_bytes(ns), stream) != hipSuccess) {
            (void)hipFree(p);
            return GEMM_RELU_EHIP;
        }
        // the old buffer stays allocated: earlier launches on this stream and
        // graphs captured from them may still use it
        if (w.base != nullptr) g_ws_retired.push_back(w.base);
        w.base = p;
        w.counter_slots = ns;
        w.partial_bytes = np;
    }
    *counters = reinterpret_cast<uint32_t*>(w.base);
    *partial = reinterpret_cast<float*>(w.base + counter_bytes(w.counter_slots));
    return GEMM_RELU_OK;
}

bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes)
{
    if (pbytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)pbytes;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)qbytes;
    return a0 < b1 && b0 < a1;
}

int validate(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* C,
             const gemm_relu_opts* opts)
{
    if (M < 0 || N < 0 || K < 0) return GEMM_RELU_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return GEMM_RELU_EUNSUPPORTED;
    // each product is below 2^62, so no overflow in int64
    const int64_t na = M * K, nb = K * N, nc = M * N;
    if ((na > 0 && !A) || (nb > 0 && !B) || (nc > 0 && !C)) return GEMM_RELU_EINVAL;
    if ((((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 1u) != 0) return GEMM_RELU_EUNSUPPORTED;
    if (overlaps(C, 2 * nc, A, 2 * na) || overlaps(C, 2 * nc, B, 2 * nb)) return GEMM_RELU_EINVAL;
    if (opts) {
        if (opts->tile != GEMM_RELU_TILE_AUTO && (opts->tile < 0 || opts->tile >= kNumTiles))
            return GEMM_RELU_EUNSUPPORTED;
        if (opts->block_order != GEMM_RELU_ORDER_DEFAULT && opts->block_order != GEMM_RELU_ORDER_ROW_MAJOR)
            return GEMM_RELU_EINVAL;
        if (opts->group_m < 0) return GEMM_RELU_EINVAL;
        for (int r : opts->reserved)
            if (r != 0) return GEMM_RELU_EINVAL;
    }
    return GEMM_RELU_OK;
}

// The bias of the bias + GELU epilogue: N fp16 values, 2-byte aligned, not
// overlapping C.
int validate_bias(int64_t M, int64_t N, const void* bias, const void* C)
{
    if (N > 0 && !bias) return GEMM_RELU_EINVAL;
    if (((uintptr_t)bias & 1u) != 0) return GEMM_RELU_EUNSUPPORTED;
    if (M > 0 && overlaps(C, 2 * M * N, bias, 2 * N)) return GEMM_RELU_EINVAL;
    return GEMM_RELU_OK;
}

// gfx950 check, once per device id.
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
signed char g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device(int& dev)
{
    dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_RELU_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_RELU_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_RELU_EHIP;
        g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    return g_dev_ok[dev] == 1 ? GEMM_RELU_OK : GEMM_RELU_EUNSUPPORTED;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: one array per GPU, in the
// library's code object, holding the split-K counters and partial sums that
// the per-stream workspaces hold for the other entry points. Its host-side
// name is only a stand-in for the device symbol: host code uses the device
// address that hipGetSymbolAddress returns for the current device, resolved
// once per device.
// ---------------------------------------------------------------------------

constexpr size_t kStaticCounterSlots = GEMM_RELU_NOALLOC_MAX_TILES;
constexpr size_t kStaticPartialBytes = GEMM_RELU_NOALLOC_MAX_PARTIAL_BYTES;
static_assert(kStaticCounterSlots * 4 % 256 == 0, "the partial sums start 256-byte aligned");
static __device__ __align__(256) char scratch[kStaticCounterSlots * 4 + kStaticPartialBytes];

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (null until resolved)

__global__ void zero_words(uint32_t* p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The current device's scratch: counters first, then the partial sums. The
// first call on a device resolves the address and clears the counters with a
// kernel on `stream` (the array is zero when the code object loads; a kernel
// rather than a memset, so that a stream under graph capture may make the
// first call). Every split-K launch leaves the counters it used at zero.
int static_scratch(int dev, hipStream_t stream, uint32_t** counters, float** partial)
{
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return GEMM_RELU_EHIP;
        }
        hipLaunchKernelGGL(zero_words, dim3((unsigned)((kStaticCounterSlots + 255) / 256)), dim3(256), 0, stream,
                           static_cast<uint32_t*>(p), (int)kStaticCounterSlots);
        if (hipGetLastError() != hipSuccess) return GEMM_RELU_EHIP;
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    *counters = reinterpret_cast<uint32_t*>(g_scratch_ptr[dev]);
    *partial = reinterpret_cast<float*>(g_scratch_ptr[dev] + kStaticCounterSlots * 4);
    return GEMM_RELU_OK;
}

// Where a split-K launch keeps its partial sums and counters.
enum class Scratch {
    kStreamWorkspace,  // the library-allocated per-(device, stream) workspace
    kStatic,           // the fixed per-device array above (allocates nothing)
};

#ifdef GR_STAMPS
// The timestamp build's buffer: kStampWords words per workgroup for launches
// of at most g_stamp_max_wg workgroups (larger launches record nothing).
uint64_t* g_stamp_buf = nullptr;
int64_t g_stamp_max_wg = 0;
#endif

// Validated call -> tile choice, split-K workspace, launch. `act` selects the
// epilogue (kActRelu, or kActBiasGelu with `bias`).
int run(int64_t M, int64_t N, int64_t K, const void* A, int op_a, const void* B, int op_b, void* C, void* stream,
        const gemm_relu_opts* opts, int act, const void* bias, Scratch where = Scratch::kStreamWorkspace)
{
    if ((op_a != GEMM_RELU_OP_N && op_a != GEMM_RELU_OP_T) || (op_b != GEMM_RELU_OP_N && op_b != GEMM_RELU_OP_T))
        return GEMM_RELU_EINVAL;
    const bool ta = op_a == GEMM_RELU_OP_T, tb = op_b == GEMM_RELU_OP_T;
    int rc = validate(M, N, K, A, B, C, opts);
    if (rc != GEMM_RELU_OK) return rc;
    if (act == gemm_relu::kActBiasGelu) {
        rc = validate_bias(M, N, bias, C);
        if (rc != GEMM_RELU_OK) return rc;
    }
    if (M == 0 || N == 0) return GEMM_RELU_OK;

    const bool vec = fast_path_ok(M, N, K, ta, tb, A, B, C);
    const int tile =
        (opts && opts->tile != GEMM_RELU_TILE_AUTO) ? opts->tile : (vec ? choose_tile(M, N, K, ta, tb) : kGenericTile);
    // the split-K tiles have no element-wise instance: unaligned shapes take
    // the generic tile
    const TileEntry& te = (!vec && kTiles[tile].desc.split_k) ? kTiles[kGenericTile] : kTiles[tile];
    const bool splitk = vec && te.desc.split_k;
    if (splitk && !splitk_ok(M, K)) return GEMM_RELU_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Args a;
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = static_cast<uint16_t*>(C);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)((M + te.desc.bm - 1) / te.desc.bm);
    a.tiles_n = (int)((N + te.desc.bn - 1) / te.desc.bn);
    if (opts && opts->group_m > 0) {
        a.group_m = opts->group_m;
        // a group of more tile-rows than there are is the same order as one
        // of all of them; clamping also keeps group_m * tiles_n within int32
        // in the kernels' block-order arithmetic
        if (a.group_m > a.tiles_m) a.group_m = a.tiles_m;
    } else {
        a.group_m = default_group(te.desc.default_group_m, a.tiles_m);
    }
    a.order = opts ? opts->block_order : GEMM_RELU_ORDER_DEFAULT;
    if (a.order == GEMM_RELU_ORDER_DEFAULT && !(opts && opts->group_m > 0))
        a.order = default_order(te.desc, a.tiles_m, a.tiles_n);
    a.trans_a = ta ? 1 : 0;
    a.trans_b = tb ? 1 : 0;
    a.act = act;
    a.bias = static_cast<const uint16_t*>(bias);
    a.partial = nullptr;
    a.counters = nullptr;
    a.splits = 1;
    a.kc = (int)(K < 1 ? 1 : K);
    a.stamps = nullptr;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles > INT32_MAX) return GEMM_RELU_EUNSUPPORTED;
    if (splitk) {
        choose_splits(M, N, K, tiles, a.splits, a.kc);
        if (tiles * a.splits > INT32_MAX) return GEMM_RELU_EUNSUPPORTED;
    }
    const size_t partial_bytes = (size_t)a.splits * (size_t)M * (size_t)N * 4;
    const bool needs_scratch = splitk && a.splits > 1;
    if (needs_scratch && where == Scratch::kStatic &&
        ((size_t)tiles > kStaticCounterSlots || partial_bytes > kStaticPartialBytes))
        return GEMM_RELU_ETOOBIG;
    int dev = 0;
    rc = check_device(dev);
    if (rc != GEMM_RELU_OK) return rc;
    if (needs_scratch) {
        rc = where == Scratch::kStatic ? static_scratch(dev, s, &a.counters, &a.partial)
                                       : get_workspace(dev, s, (size_t)tiles, partial_bytes, &a.counters, &a.partial);
        if (rc != GEMM_RELU_OK) return rc;
    }
#ifdef GR_STAMPS
    if (tiles * a.splits <= g_stamp_max_wg) a.stamps = g_stamp_buf;
#endif
    const hipError_t e = (vec ? te.vec : te.generic)(a, s);
    return e == hipSuccess ? GEMM_RELU_OK : GEMM_RELU_EHIP;
}

}  // namespace

extern "C" {

const char* gemm_relu_strerror(int status)
{
    switch (status) {
    case GEMM_RELU_OK: return "success";
    case GEMM_RELU_EINVAL: return "invalid argument (negative size, NULL pointer, or C overlapping A/B)";
    case GEMM_RELU_EUNSUPPORTED: return "unsupported (size above INT32_MAX, misaligned pointer, device not gfx950, or unknown tile)";
    case GEMM_RELU_EHIP: return "HIP runtime error";
    case GEMM_RELU_ENOMEM: return "workspace allocation failed";
    case GEMM_RELU_ETOOBIG:
        return "the split-K launch needs more scratch than the allocation-free entry point holds "
               "(more than GEMM_RELU_NOALLOC_MAX_TILES output tiles or GEMM_RELU_NOALLOC_MAX_PARTIAL_BYTES of partial sums)";
    default: return "unknown status";
    }
}

#ifdef GR_STAMPS
// Timestamp build only (not part of the ABI in include/): device buffer of
// max_workgroups * 8 words that later launches fill, one row per workgroup
// (see GR_STAMP_FLUSH in common.hpp); NULL or 0 turns recording off.
int gemm_relu_stamps_set(void* buf, int64_t max_workgroups)
{
    g_stamp_buf = static_cast<uint64_t*>(buf);
    g_stamp_max_wg = buf ? max_workgroups : 0;
    return GEMM_RELU_OK;
}
#endif

int gemm_relu_tile_count(void) { return kNumTiles; }

const char* gemm_relu_tile_name(int tile)
{
    return (tile >= 0 && tile < kNumTiles) ? kTiles[tile].name : "";
}

int gemm_relu_tile_info(int tile, gemm_relu_tile_desc* desc)
{
    if (!desc) return GEMM_RELU_EINVAL;
    if (tile < 0 || tile >= kNumTiles) return GEMM_RELU_EUNSUPPORTED;
    *desc = kTiles[tile].desc;
    return GEMM_RELU_OK;
}

int gemm_relu_default_order(int tile, int64_t M, int64_t N, int32_t* block_order, int32_t* group_m)
{
    if (!block_order || !group_m || M < 0 || N < 0) return GEMM_RELU_EINVAL;
    if (tile < 0 || tile >= kNumTiles) return GEMM_RELU_EUNSUPPORTED;
    const gemm_relu_tile_desc& d = kTiles[tile].desc;
    const int64_t tiles_m = (M + d.bm - 1) / d.bm, tiles_n = (N + d.bn - 1) / d.bn;
    *group_m = default_group(d.default_group_m, (int)(tiles_m < INT32_MAX ? tiles_m : INT32_MAX));
    *block_order = default_order(d, tiles_m, tiles_n);
    return GEMM_RELU_OK;
}

int gemm_relu_select_tile(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* C)
{
    return gemm_relu_select_tile_op(M, N, K, GEMM_RELU_OP_N, GEMM_RELU_OP_N, A, B, C);
}

int gemm_relu_select_tile_op(int64_t M, int64_t N, int64_t K, int op_a, int op_b, const void* A, const void* B,
                             const void* C)
{
    if ((op_a != GEMM_RELU_OP_N && op_a != GEMM_RELU_OP_T) || (op_b != GEMM_RELU_OP_N && op_b != GEMM_RELU_OP_T))
        return -1;
    const bool ta = op_a == GEMM_RELU_OP_T, tb = op_b == GEMM_RELU_OP_T;
    if (!fast_path_ok(M, N, K, ta, tb, A, B, C)) return -1;
    return choose_tile(M, N, K, ta, tb);
}

int gemm_relu_f16_ex(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C,
                     void* stream, const gemm_relu_opts* opts)
{
    return run(M, N, K, A, GEMM_RELU_OP_N, B, GEMM_RELU_OP_N, C, stream, opts, gemm_relu::kActRelu, nullptr);
}

int gemm_relu_f16(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, void* stream)
{
    return run(M, N, K, A, GEMM_RELU_OP_N, B, GEMM_RELU_OP_N, C, stream, nullptr, gemm_relu::kActRelu, nullptr);
}

int gemm_relu_f16_noalloc(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, void* stream)
{
    return run(M, N, K, A, GEMM_RELU_OP_N, B, GEMM_RELU_OP_N, C, stream, nullptr, gemm_relu::kActRelu, nullptr,
               Scratch::kStatic);
}

int gemm_relu_f16_op(int64_t M, int64_t N, int64_t K, const void* A, int op_a, const void* B, int op_b, void* C,
                     void* stream, const gemm_relu_opts* opts)
{
    return run(M, N, K, A, op_a, B, op_b, C, stream, opts, gemm_relu::kActRelu, nullptr);
}

int gemm_bias_gelu_f16_ex(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                          void* C, void* stream, const gemm_relu_opts* opts)
{
    return run(M, N, K, A, GEMM_RELU_OP_N, B, GEMM_RELU_OP_N, C, stream, opts, gemm_relu::kActBiasGelu, bias);
}

int gemm_bias_gelu_f16(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* bias,
                       void* C, void* stream)
{
    return run(M, N, K, A, GEMM_RELU_OP_N, B, GEMM_RELU_OP_N, C, stream, nullptr, gemm_relu::kActBiasGelu, bias);
}

int gemm_bias_gelu_f16_op(int64_t M, int64_t N, int64_t K, const void* A, int op_a, const void* B, int op_b,
                          const void* bias, void* C, void* stream, const gemm_relu_opts* opts)
{
    return run(M, N, K, A, op_a, B, op_b, C, stream, opts, gemm_relu::kActBiasGelu, bias);
}

}  // extern "C"

// C = ReLU(A @ B) for fp16 A[M,K], B[K,N] on MI355X (gfx950, CDNA4): the
// host side of the C ABI declared in include/gemm_relu.h.
//
// The computation is the GEMM + ReLU example of "Writing high-performance
// kernels in TileLang" (section "Escribamos un GEMM"). Two kernel families
// implement it:
//  * pipelined.hpp -- the large-tile hot path: direct-to-LDS loads, a
//    four-stage LDS ring, v_mfma_f32_32x32x16_f16, transposing LDS reads;
//  * staged.hpp    -- register-staged loads with v_mfma_f32_16x16x32_f16, for
//    small tiles and for the generic element-wise path (any K, N, alignment).
// This file holds the tile table, the shape heuristic, argument validation
// and the launches.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "gemm_relu.h"
#include "pipelined.hpp"
#include "staged.hpp"

namespace {

// ---------------------------------------------------------------------------
// Tile table
// ---------------------------------------------------------------------------

using gemm_relu::Args;

using P256 = gemm_relu::pipelined::Cfg<256, 256, 2, 2>;   // 4 waves x 128x128, 32x32x16 MFMA
using S256 = gemm_relu::staged::Tile<256, 256, 64, 2, 2>;  // generic instance of the same tile
using S128 = gemm_relu::staged::Tile<128, 128, 64, 2, 2>;  // the pages' 128x128x64 tile
using S64 = gemm_relu::staged::Tile<64, 64, 64, 2, 2>;     // 4 waves x 32x32
using S16 = gemm_relu::staged::Tile<16, 64, 64, 1, 4>;     // 4 waves x 16x16: few rows

using LaunchFn = hipError_t (*)(const Args&, hipStream_t);

template <class T, bool VEC>
hipError_t launch_staged(const Args& a, hipStream_t s)
{
    const int blocks = a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((gemm_relu::staged::staged_kernel<T, VEC>), dim3(blocks), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

template <class T>
hipError_t launch_pipelined(const Args& a, hipStream_t s)
{
    const int blocks = a.tiles_m * a.tiles_n;
    if (a.K % T::BK == 0)
        hipLaunchKernelGGL((gemm_relu::pipelined::pipelined_kernel<T, true>), dim3(blocks), dim3(T::NT), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_relu::pipelined::pipelined_kernel<T, false>), dim3(blocks), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

struct TileEntry {
    const char* name;
    int bm, bn;
    int default_group_m;
    LaunchFn vec;
    LaunchFn generic;
};

const TileEntry kTiles[] = {
    {"256x256x32s4_w2x2_mfma32x32x16_lds-dma", 256, 256, 4, launch_pipelined<P256>, launch_staged<S256, false>},
    {"128x128x64_w2x2_mfma16x16x32", 128, 128, 4, launch_staged<S128, true>, launch_staged<S128, false>},
    {"64x64x64_w2x2_mfma16x16x32", 64, 64, 4, launch_staged<S64, true>, launch_staged<S64, false>},
    {"16x64x64_w1x4_mfma16x16x32", 16, 64, 1, launch_staged<S16, true>, launch_staged<S16, false>},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kGenericTile = 2;  // tile used by the element-wise path

bool fast_path_ok(int64_t N, int64_t K, const void* A, const void* B, const void* C)
{
    const uintptr_t mis = ((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15u;
    // 32-bit in-tile buffer offsets: BM*K*2 and BK*N*2 must stay below 2^31
    return (K % 8 == 0) && (N % 8 == 0) && mis == 0 && K <= (1 << 22) && N <= (1 << 24);
}

int choose_tile(int64_t M, int64_t N)
{
    auto blocks = [&](int t) {
        return ((M + kTiles[t].bm - 1) / kTiles[t].bm) * ((N + kTiles[t].bn - 1) / kTiles[t].bn);
    };
    if (M <= 16) return 3;
    if (blocks(0) >= 256) return 0;
    if (blocks(1) >= 128) return 1;
    return 2;
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

// gfx950 check, once per device id.
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
signed char g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device()
{
    int dev = 0;
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
    default: return "unknown status";
    }
}

int gemm_relu_tile_count(void) { return kNumTiles; }

const char* gemm_relu_tile_name(int tile)
{
    return (tile >= 0 && tile < kNumTiles) ? kTiles[tile].name : "";
}

int gemm_relu_select_tile(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* C)
{
    if (!fast_path_ok(N, K, A, B, C)) return -1;
    return choose_tile(M, N);
}

int gemm_relu_f16_ex(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C,
                     void* stream, const gemm_relu_opts* opts)
{
    int rc = validate(M, N, K, A, B, C, opts);
    if (rc != GEMM_RELU_OK) return rc;
    if (M == 0 || N == 0) return GEMM_RELU_OK;
    rc = check_device();
    if (rc != GEMM_RELU_OK) return rc;

    const bool vec = fast_path_ok(N, K, A, B, C);
    int tile = (opts && opts->tile != GEMM_RELU_TILE_AUTO) ? opts->tile : (vec ? choose_tile(M, N) : kGenericTile);
    const TileEntry& te = kTiles[tile];
    Args a;
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = static_cast<uint16_t*>(C);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)((M + te.bm - 1) / te.bm);
    a.tiles_n = (int)((N + te.bn - 1) / te.bn);
    a.group_m = (opts && opts->group_m > 0) ? opts->group_m : te.default_group_m;
    a.order = opts ? opts->block_order : GEMM_RELU_ORDER_DEFAULT;
    if ((int64_t)a.tiles_m * a.tiles_n > INT32_MAX) return GEMM_RELU_EUNSUPPORTED;
    const hipError_t e = (vec ? te.vec : te.generic)(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_RELU_OK : GEMM_RELU_EHIP;
}

int gemm_relu_f16(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, void* stream)
{
    return gemm_relu_f16_ex(M, N, K, A, B, C, stream, nullptr);
}

}  // extern "C"

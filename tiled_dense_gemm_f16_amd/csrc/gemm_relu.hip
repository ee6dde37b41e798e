// C = ReLU(A @ B) for fp16 A[M,K], B[K,N] on MI355X (gfx950, CDNA4).
//
// The computation is the GEMM + ReLU example of "Writing high-performance
// kernels in TileLang" (section "Escribamos un GEMM"): each workgroup owns one
// BM x BN tile of C, walks K in BK-wide steps that are staged through shared
// memory (LDS here), keeps the tile's accumulator in registers in fp32, then
// applies max(x, 0) and stores fp16. The pieces map onto CDNA4 as follows:
//
//  * tile products run on the matrix cores: v_mfma_f32_16x16x32_f16, one
//    64-lane wave per WM x WN sub-tile (the pages' warp policy becomes a fixed
//    wave grid inside the workgroup);
//  * global -> LDS copies are 16-byte buffer loads (out-of-range lanes are
//    given an offset past the buffer's end, so the hardware returns zeros --
//    this is the edge masking of the ragged tiles);
//  * A is stored k-contiguous ([BM][BK]); B arrives n-contiguous and is
//    transposed in registers (8x8 blocks of halves) so that it is also stored
//    k-contiguous ([BN][BK]); both use an XOR swizzle of the 16-byte chunk
//    index against the row, so the MFMA fragment reads hit distinct banks;
//  * two LDS stages plus a register prefetch give a three-deep pipeline (the
//    pages' num_stages = 3): tile k+1 is in flight from HBM while tile k is
//    multiplied, and k+1 is written to the other LDS stage before the barrier;
//  * the tile order is remapped per XCD (each of the 8 dies has its own L2,
//    and the hardware deals workgroups round-robin over the dies) and grouped
//    by tile-rows, the counterpart of the pages' L2 swizzle of block order;
//  * the epilogue applies ReLU to the fp32 accumulators and converts with
//    v_cvt_f16_f32 (round to nearest even), then stores 8 bytes per lane.
//
// A generic instance of the same kernel loads element by element; it serves
// shapes whose K or N is not a multiple of 8 or whose pointers are not 16-byte
// aligned.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "gemm_relu.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// An offset that is never inside a buffer: every buffer is given at most this
// many records, so a lane loading here reads zeros.
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

// 16-byte chunk swizzle for a row of 8 chunks (BK = 64 halves): XOR with the
// row's low three bits, so 8 consecutive rows read at one logical chunk land
// on 8 different physical chunks (all 32 four-byte banks of a 128-byte span).
__device__ __forceinline__ int swz(int row) { return row & 7; }

// Maps the launch index to a (tile_m, tile_n) pair.
//  1. XCD remap: workgroup b is dispatched to die b % 8. Renumber so that die
//     x receives one contiguous range of tile ids (a bijection for any count).
//  2. Grouped order: ids run down `group_m` tile-rows before moving to the next
//     tile-column, so tiles that run together share A row-panels and B
//     column-panels in that die's L2.
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

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MIN_WAVES_ = 1>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = kWave * WAVES_M * WAVES_N;
    static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // per-wave sub-tile
    static constexpr int FM = TM / 16, FN = TN / 16;              // 16x16 MFMA blocks
    static constexpr int KC = BK / 8;                             // 16-byte chunks per row
    static constexpr int A_CHUNKS = BM * KC;                      // per stage
    static constexpr int B_UNITS = KC * (BN / 8);                 // 8x8 blocks per stage
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_PER_T = (B_UNITS + NT - 1) / NT;
    static constexpr int STAGE_HALVES = (BM + BN) * BK;
    static constexpr int LDS_BYTES = 2 * STAGE_HALVES * 2;
    static constexpr int MIN_WAVES = MIN_WAVES_;
    static_assert(BK == 64, "the swizzle assumes 8 chunks per row");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole MFMA blocks");
    static_assert(BM % WAVES_M == 0 && BN % WAVES_N == 0, "waves must divide the tile");
};

// Registers holding one k-step of the block's operands on their way to LDS.
template <class T>
struct Staging {
    u32x4 a[T::A_PER_T];
    u32x4 b[T::B_PER_T][8];
};

template <class T, bool VEC>
__device__ __forceinline__ void load_tile(const Args& p, int m0, int n0, int k0, Staging<T>& st)
{
    const int t = threadIdx.x;
    const int K = p.K, N = p.N, M = p.M;
    if constexpr (VEC) {
        // A: BM rows x KC chunks, block base at row m0, column k0
        const uint16_t* abase = p.A + (int64_t)m0 * K + k0;
        const uint64_t arem = ((uint64_t)(M - m0) * (uint64_t)K - (uint64_t)k0) * 2u;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase, arem);
        const bool ktail = (k0 + T::BK > K);
#pragma unroll
        for (int i = 0; i < T::A_PER_T; ++i) {
            const int c = t + i * T::NT;
            const int row = c / T::KC, kc = c % T::KC;
            bool ok = (c < T::A_CHUNKS) && (m0 + row < M);
            if (ktail) ok = ok && (k0 + kc * 8 < K);
            const uint32_t off = ok ? (uint32_t)(row * K + kc * 8) * 2u : kOOB;
            st.a[i] = load16(ra, off);
        }
        // B: BK rows x BN columns as 8x8 units; unit u -> k-block u % KC,
        // n-block u / KC (8 consecutive lanes cover one n-block's 8 k-blocks,
        // so the transposed LDS writes below hit 8 different chunks)
        const uint16_t* bbase = p.B + (int64_t)k0 * N;
        const uint64_t brem = (uint64_t)(K - k0) * (uint64_t)N * 2u;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bbase, brem);
#pragma unroll
        for (int i = 0; i < T::B_PER_T; ++i) {
            const int u = t + i * T::NT;
            const int kb = u % T::KC, nb = u / T::KC;
            const bool uok = (u < T::B_UNITS) && (n0 + nb * 8 < N);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int kr = kb * 8 + r;
                const bool ok = uok && (!ktail || k0 + kr < K);
                const uint32_t off = ok ? (uint32_t)(kr * N + n0 + nb * 8) * 2u : kOOB;
                st.b[i][r] = load16(rb, off);
            }
        }
    } else {
        // element-wise loads with full bounds checks (any K, N, alignment)
#pragma unroll
        for (int i = 0; i < T::A_PER_T; ++i) {
            const int c = t + i * T::NT;
            const int row = c / T::KC, kc = c % T::KC;
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int gm = m0 + row, gk = k0 + kc * 8 + e;
                h[e] = (c < T::A_CHUNKS && gm < M && gk < K) ? p.A[(int64_t)gm * K + gk] : (uint16_t)0;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) st.a[i][j] = (uint32_t)h[2 * j] | ((uint32_t)h[2 * j + 1] << 16);
        }
#pragma unroll
        for (int i = 0; i < T::B_PER_T; ++i) {
            const int u = t + i * T::NT;
            const int kb = u % T::KC, nb = u / T::KC;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                uint16_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int gk = k0 + kb * 8 + r, gn = n0 + nb * 8 + e;
                    h[e] = (u < T::B_UNITS && gk < K && gn < N) ? p.B[(int64_t)gk * N + gn] : (uint16_t)0;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) st.b[i][r][j] = (uint32_t)h[2 * j] | ((uint32_t)h[2 * j + 1] << 16);
            }
        }
    }
}

template <class T>
__device__ __forceinline__ void store_tile(uint16_t* As, uint16_t* Bs, const Staging<T>& st)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
        const int c = t + i * T::NT;
        if (c < T::A_CHUNKS) {
            const int row = c / T::KC, kc = c % T::KC;
            *reinterpret_cast<u32x4*>(As + row * T::BK + ((kc ^ swz(row)) * 8)) = st.a[i];
        }
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_T; ++i) {
        const int u = t + i * T::NT;
        if (u < T::B_UNITS) {
            const int kb = u % T::KC, nb = u / T::KC;
            u32x4 cols[8];
            transpose8x8(st.b[i], cols);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int n = nb * 8 + c;
                *reinterpret_cast<u32x4*>(Bs + n * T::BK + ((kb ^ swz(n)) * 8)) = cols[c];
            }
        }
    }
}

template <class T>
__device__ __forceinline__ void compute_tile(const uint16_t* As, const uint16_t* Bs,
                                             f32x4 (&acc)[T::FM][T::FN], int wm, int wn, int lane)
{
    const int lr = lane & 15;  // row (A) / column (B) of the 16-wide fragment
    const int lg = lane >> 4;  // which 8-wide k-slice of the 32-deep step
#pragma unroll
    for (int kk = 0; kk < T::BK / 32; ++kk) {
        const int c = kk * 4 + lg;
        f16x8 af[T::FM], bf[T::FN];
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm) {
            const int r = wm * T::TM + fm * 16 + lr;
            af[fm] = *reinterpret_cast<const f16x8*>(As + r * T::BK + ((c ^ swz(r)) * 8));
        }
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            const int n = wn * T::TN + fn * 16 + lr;
            bf[fn] = *reinterpret_cast<const f16x8*>(Bs + n * T::BK + ((c ^ swz(n)) * 8));
        }
        // B fragment as the first operand: the result block is C^T, so each
        // lane ends up holding 4 consecutive columns of one row of C.
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[fn], af[fm], acc[fm][fn], 0, 0, 0);
    }
}

template <class T, bool VEC>
__global__ void __launch_bounds__(T::NT, T::MIN_WAVES) gemm_relu_kernel(Args p)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE_HALVES];

    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    f32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (p.K + T::BK - 1) / T::BK;
    Staging<T> st;
    if (nk > 0) {
        load_tile<T, VEC>(p, m0, n0, 0, st);
        store_tile<T>(smem, smem + T::BM * T::BK, st);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        uint16_t* cur = smem + (kt & 1) * T::STAGE_HALVES;
        uint16_t* nxt = smem + ((kt + 1) & 1) * T::STAGE_HALVES;
        const bool more = kt + 1 < nk;
        if (more) load_tile<T, VEC>(p, m0, n0, (kt + 1) * T::BK, st);
        compute_tile<T>(cur, cur + T::BM * T::BK, acc, wm, wn, lane);
        if (more) store_tile<T>(nxt, nxt + T::BM * T::BK, st);
        __syncthreads();
    }

    // Epilogue: ReLU on the fp32 accumulator, round to fp16 (nearest even),
    // store. Lane holds rows m, columns n .. n+3 of each 16x16 block.
    const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm) {
        const int m = m0 + wm * T::TM + fm * 16 + lr;
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            const int n = n0 + wn * T::TN + fn * 16 + lg * 4;
            _Float16 h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = (_Float16)fmaxf(acc[fm][fn][r], 0.0f);
            if (m < p.M) {
                uint16_t* dst = p.C + (int64_t)m * p.N + n;
                if constexpr (VEC) {
                    if (n < p.N) {
                        u32x2 v;
                        v[0] = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
                        v[1] = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
                        *reinterpret_cast<u32x2*>(dst) = v;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < p.N) dst[r] = __builtin_bit_cast(uint16_t, h[r]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tile table
// ---------------------------------------------------------------------------

using Tile256 = Tile<256, 256, 64, 2, 2>;  // 4 waves x 128x128: the large-problem tile
using Tile128 = Tile<128, 128, 64, 2, 2>;  // 4 waves x 64x64: the pages' 128x128x64 tile
using Tile64 = Tile<64, 64, 64, 2, 2>;     // 4 waves x 32x32
using Tile16 = Tile<16, 64, 64, 1, 4>;     // 4 waves x 16x16: few rows (decode-like)

using LaunchFn = hipError_t (*)(const Args&, hipStream_t);

template <class T, bool VEC>
hipError_t launch(const Args& a, hipStream_t s)
{
    const int blocks = a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((gemm_relu_kernel<T, VEC>), dim3(blocks), dim3(T::NT), 0, s, a);
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
    {"256x256x64_w2x2_mfma16x16x32", 256, 256, 4, launch<Tile256, true>, launch<Tile256, false>},
    {"128x128x64_w2x2_mfma16x16x32", 128, 128, 4, launch<Tile128, true>, launch<Tile128, false>},
    {"64x64x64_w2x2_mfma16x16x32", 64, 64, 4, launch<Tile64, true>, launch<Tile64, false>},
    {"16x64x64_w1x4_mfma16x16x32", 16, 64, 1, launch<Tile16, true>, launch<Tile16, false>},
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

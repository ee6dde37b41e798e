// Register-staged kernel: the first, general-purpose instance of the tiled
// GEMM + ReLU. It serves small tiles and the generic element-wise path.
//
// Each workgroup owns one BM x BN tile of C and walks K in BK = 64 steps:
//  * 16-byte buffer loads bring the next A and B tiles into registers while
//    the current tile is multiplied (out-of-range lanes read zeros);
//  * A is stored k-contiguous ([BM][BK]); B arrives n-contiguous and is
//    transposed in registers (8x8 blocks of halves) so it is also stored
//    k-contiguous ([BN][BK]); both use an XOR swizzle of the 16-byte chunk
//    index, so fragment reads hit distinct LDS banks. Transposed operands
//    (A given as K x M, B as N x K) swap which of the two load paths each
//    operand takes; the LDS tiles and everything after them are the same;
//  * two LDS stages plus the register prefetch form a three-deep pipeline;
//  * tile products run on v_mfma_f32_16x16x32_f16 with the B fragment as the
//    first operand, so the result block is C^T and each lane holds four
//    consecutive columns of one row -- the epilogue stores 8 bytes per lane.
// With VEC = false every global access is an element-wise, bounds-checked
// load or store: any K, N and pointer alignment.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace gemm_relu {
namespace staged {

// 16-byte chunk swizzle for a row of 8 chunks (BK = 64 halves): XOR with the
// row's low three bits, so 8 consecutive rows read at one logical chunk land
// on 8 different physical chunks (all 32 four-byte banks of a 128-byte span).
__device__ __forceinline__ int swz(int row) { return row & 7; }

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MIN_WAVES_ = 1, int PREFETCH_ = 1>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = kWave * WAVES_M * WAVES_N;
    static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // per-wave sub-tile
    static constexpr int FM = TM / 16, FN = TN / 16;              // 16x16 MFMA blocks
    static constexpr int KC = BK / 8;                             // 16-byte chunks per row
    static constexpr int STAGE_HALVES = (BM + BN) * BK;
    static constexpr int LDS_BYTES = 2 * STAGE_HALVES * 2;
    static constexpr int MIN_WAVES = MIN_WAVES_;
    // k-steps whose loads are in flight in registers (vector path only)
    static constexpr int PREFETCH = PREFETCH_;
    static_assert(PREFETCH >= 1 && PREFETCH <= 8, "register ring depth");
    static_assert(BK == 64, "the swizzle assumes 8 chunks per row");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole MFMA blocks");
    static_assert(BM % WAVES_M == 0 && BN % WAVES_N == 0, "waves must divide the tile");
};

// Registers holding one k-step of one operand on its way to LDS. An operand
// stored k-contiguous (A as given, or B given as N x K) arrives as 16-byte
// chunks of 8 consecutive k; one stored mn-contiguous (B as given, or A given
// as K x M) arrives as 8 x 8 blocks (8 k-rows of 8 columns), transposed in
// registers before the LDS write. Either way the LDS tile is [ROWS][BK].
template <class T, int ROWS>
struct KChunks {
    static constexpr int COUNT = ROWS * T::KC;
    static constexpr int PER_T = (COUNT + T::NT - 1) / T::NT;
    u32x4 v[PER_T];
};

template <class T, int ROWS>
struct MNUnits {
    static constexpr int COUNT = T::KC * (ROWS / 8);
    static constexpr int PER_T = (COUNT + T::NT - 1) / T::NT;
    u32x4 v[PER_T][8];
};

template <class T, bool TA, bool TB>
struct Staging {
    std::conditional_t<TA, MNUnits<T, T::BM>, KChunks<T, T::BM>> a;
    std::conditional_t<TB, KChunks<T, T::BN>, MNUnits<T, T::BN>> b;
};

// Rows [row0, row0 + ROWS) and k-columns [k0, k0 + BK) of a k-contiguous
// operand X[rows_total][K]. Chunk c of the tile is row c / KC, k-chunk c % KC.
template <class T, int ROWS, bool VEC>
__device__ __forceinline__ void load_k(const uint16_t* X, int rows_total, int row0, int k0, int K,
                                       KChunks<T, ROWS>& st)
{
    using S = KChunks<T, ROWS>;
    const int t = threadIdx.x;
    if constexpr (VEC) {
        // a step past the end of K gets an empty descriptor: zeros
        const int64_t rem = ((int64_t)(rows_total - row0) * K - k0) * 2;
        const uint16_t* base = X + (int64_t)row0 * K + (k0 < K ? k0 : K);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint64_t)(k0 < K && rem > 0 ? rem : 0));
        const bool ktail = (k0 + T::BK > K);
#pragma unroll
        for (int i = 0; i < S::PER_T; ++i) {
            const int c = t + i * T::NT;
            const int row = c / T::KC, kc = c % T::KC;
            bool ok = (c < S::COUNT) && (row0 + row < rows_total);
            if (ktail) ok = ok && (k0 + kc * 8 < K);
            st.v[i] = load16(r, ok ? (uint32_t)(row * K + kc * 8) * 2u : kOOB);
        }
    } else {
        // element-wise loads with full bounds checks (any K, N, alignment)
#pragma unroll
        for (int i = 0; i < S::PER_T; ++i) {
            const int c = t + i * T::NT;
            const int row = c / T::KC, kc = c % T::KC;
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int gr = row0 + row, gk = k0 + kc * 8 + e;
                h[e] = (c < S::COUNT && gr < rows_total && gk < K) ? X[(int64_t)gr * K + gk] : (uint16_t)0;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) st.v[i][j] = (uint32_t)h[2 * j] | ((uint32_t)h[2 * j + 1] << 16);
        }
    }
}

// k-rows [k0, k0 + BK) and columns [row0, row0 + ROWS) of an mn-contiguous
// operand X[K][ld]. Unit u is k-block u % KC, column block u / KC (8
// consecutive threads cover one column block's k-blocks, so the transposed
// LDS writes hit 8 different chunks).
template <class T, int ROWS, bool VEC>
__device__ __forceinline__ void load_mn(const uint16_t* X, int ld, int row0, int k0, int K, MNUnits<T, ROWS>& st)
{
    using S = MNUnits<T, ROWS>;
    const int t = threadIdx.x;
    const bool ktail = (k0 + T::BK > K);
    if constexpr (VEC) {
        const int64_t rem = ((int64_t)K - k0) * ld * 2;
        const uint16_t* base = X + (int64_t)(k0 < K ? k0 : K) * ld;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint64_t)(rem > 0 ? rem : 0));
#pragma unroll
        for (int i = 0; i < S::PER_T; ++i) {
            const int u = t + i * T::NT;
            const int kb = u % T::KC, nb = u / T::KC;
            const bool uok = (u < S::COUNT) && (row0 + nb * 8 < ld);
#pragma unroll
            for (int r8 = 0; r8 < 8; ++r8) {
                const int kr = kb * 8 + r8;
                const bool ok = uok && (!ktail || k0 + kr < K);
                st.v[i][r8] = load16(r, ok ? (uint32_t)(kr * ld + row0 + nb * 8) * 2u : kOOB);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < S::PER_T; ++i) {
            const int u = t + i * T::NT;
            const int kb = u % T::KC, nb = u / T::KC;
#pragma unroll
            for (int r8 = 0; r8 < 8; ++r8) {
                uint16_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int gk = k0 + kb * 8 + r8, gc = row0 + nb * 8 + e;
                    h[e] = (u < S::COUNT && gk < K && gc < ld) ? X[(int64_t)gk * ld + gc] : (uint16_t)0;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) st.v[i][r8][j] = (uint32_t)h[2 * j] | ((uint32_t)h[2 * j + 1] << 16);
            }
        }
    }
}

template <class T, bool VEC, bool TA, bool TB>
__device__ __forceinline__ void load_tile(const Args& p, int m0, int n0, int k0, Staging<T, TA, TB>& st)
{
    if constexpr (TA) load_mn<T, T::BM, VEC>(p.A, p.M, m0, k0, p.K, st.a);
    else load_k<T, T::BM, VEC>(p.A, p.M, m0, k0, p.K, st.a);
    if constexpr (TB) load_k<T, T::BN, VEC>(p.B, p.N, n0, k0, p.K, st.b);
    else load_mn<T, T::BN, VEC>(p.B, p.N, n0, k0, p.K, st.b);
}

template <class T, int ROWS>
__device__ __forceinline__ void store_op(uint16_t* Xs, const KChunks<T, ROWS>& st)
{
    using S = KChunks<T, ROWS>;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < S::PER_T; ++i) {
        const int c = t + i * T::NT;
        if (c < S::COUNT) {
            const int row = c / T::KC, kc = c % T::KC;
            *reinterpret_cast<u32x4*>(Xs + row * T::BK + ((kc ^ swz(row)) * 8)) = st.v[i];
        }
    }
}

template <class T, int ROWS>
__device__ __forceinline__ void store_op(uint16_t* Xs, const MNUnits<T, ROWS>& st)
{
    using S = MNUnits<T, ROWS>;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < S::PER_T; ++i) {
        const int u = t + i * T::NT;
        if (u < S::COUNT) {
            const int kb = u % T::KC, nb = u / T::KC;
            u32x4 cols[8];
            transpose8x8(st.v[i], cols);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int n = nb * 8 + c;
                *reinterpret_cast<u32x4*>(Xs + n * T::BK + ((kb ^ swz(n)) * 8)) = cols[c];
            }
        }
    }
}

template <class T, bool TA, bool TB>
__device__ __forceinline__ void store_tile(uint16_t* As, uint16_t* Bs, const Staging<T, TA, TB>& st)
{
    store_op<T, T::BM>(As, st.a);
    store_op<T, T::BN>(Bs, st.b);
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

template <class T, bool VEC, bool TA = false, bool TB = false>
__global__ void __launch_bounds__(T::NT, T::MIN_WAVES) staged_kernel(Args p)
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
    if constexpr (!VEC || T::PREFETCH == 1) {
        Staging<T, TA, TB> st;
        if (nk > 0) {
            load_tile<T, VEC, TA, TB>(p, m0, n0, 0, st);
            store_tile<T, TA, TB>(smem, smem + T::BM * T::BK, st);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; ++kt) {
            uint16_t* cur = smem + (kt & 1) * T::STAGE_HALVES;
            uint16_t* nxt = smem + ((kt + 1) & 1) * T::STAGE_HALVES;
            const bool more = kt + 1 < nk;
            if (more) load_tile<T, VEC, TA, TB>(p, m0, n0, (kt + 1) * T::BK, st);
            compute_tile<T>(cur, cur + T::BM * T::BK, acc, wm, wn, lane);
            if (more) store_tile<T, TA, TB>(nxt, nxt + T::BM * T::BK, st);
            __syncthreads();
        }
    } else {
        // Register ring of D = PREFETCH k-steps: step s lives in slot s % D.
        // While step kt is multiplied out of LDS, step kt+1 is moved from its
        // slot into the other LDS buffer and the loads of step kt+1+D are
        // issued into the slot it frees, so D steps of loads are in flight:
        // with small tiles one step's multiply is far shorter than a load's
        // latency. The loop body has no branches (they make the compiler
        // drain every load before each LDS store): it runs for nk rounded up
        // to a multiple of D, and steps past the end of K load and multiply
        // zeros.
        constexpr int D = T::PREFETCH;
        Staging<T, TA, TB> st[D];
        auto issue = [&](int slot, int s) { load_tile<T, true, TA, TB>(p, m0, n0, s * T::BK, st[slot]); };
#pragma unroll
        for (int d = 0; d < D; ++d) {
            issue(d, d);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int nkd = (nk + D - 1) / D * D;
        if (nk > 0) {
            store_tile<T, TA, TB>(smem, smem + T::BM * T::BK, st[0]);
            __syncthreads();
            issue(0, D);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int kt0 = 0; kt0 < nkd; kt0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int kt = kt0 + d;
                uint16_t* cur = smem + (kt & 1) * T::STAGE_HALVES;
                uint16_t* nxt = smem + ((kt + 1) & 1) * T::STAGE_HALVES;
                compute_tile<T>(cur, cur + T::BM * T::BK, acc, wm, wn, lane);
                __builtin_amdgcn_sched_barrier(0);
                store_tile<T, TA, TB>(nxt, nxt + T::BM * T::BK, st[(d + 1) % D]);
                __syncthreads();
                issue((d + 1) % D, kt + 1 + D);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vmcnt<0>();  // the loads past the end must land before the kernel ends
    }

    // Epilogue: ReLU (or bias + GELU) on the fp32 accumulator, round to fp16
    // (nearest even), store. Lane holds rows m, columns n .. n+3 of each 16x16
    // block.
    const int lr = lane & 15, lg = lane >> 4;
    with_epilogue(p, [&]<int ACT>() {
        // vector path: the bias of this lane's columns, loaded once for all its rows
        f32x4 bias[T::FN];
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
            bias[fn] = (VEC && ACT == kActBiasGelu) ? bias4(p, n0 + wn * T::TN + fn * 16 + lg * 4)
                                                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm) {
            const int m = m0 + wm * T::TM + fm * 16 + lr;
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn) {
                const int n = n0 + wn * T::TN + fn * 16 + lg * 4;
                const f32x4 v = acc[fm][fn];
                if (m < p.M) {
                    uint16_t* dst = p.C + (int64_t)m * p.N + n;
                    if constexpr (VEC) {
                        if (n < p.N) {
                            u32x2 w;
                            w[0] = epi_pack2b<ACT>(v[0], v[1], bias[fn][0], bias[fn][1]);
                            w[1] = epi_pack2b<ACT>(v[2], v[3], bias[fn][2], bias[fn][3]);
                            *reinterpret_cast<u32x2*>(dst) = w;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < p.N) dst[r] = epi_f16<ACT>(p, v[r], n + r);
                    }
                }
            }
        }
    });
}

}  // namespace staged
}  // namespace gemm_relu

// Pipelined kernel for small and mid-size tiles (64 x 64 and the like): the
// tiles that fill all 256 compute units on problems of about 1024^3 and
// below, where the 256 x 256 tile of pipelined.hpp leaves most of the chip
// idle.
//
// Same computation as the TileLang GEMM + ReLU example ("Writing
// high-performance kernels in TileLang", section "Escribamos un GEMM"): a
// BM x BN tile of C per workgroup, K walked in steps staged through shared
// memory with a multi-stage software pipeline, fp32 accumulators in
// registers, max(x, 0), fp16 store. The gfx950 design:
//
//  * Direct-to-LDS loads (buffer_load_dwordx4 ... lds, 1 KiB per
//    instruction) into a ring of STAGES slots, one LDS array per slot; loads
//    for a step are issued STAGES steps ahead of the matrix ops that use it.
//    Out-of-range lanes are given an offset past the buffer's end and read
//    zeros: the masking of ragged edge tiles in M, N and the K tail.
//  * A step is BK = 32 * KSUB deep: A as [BM][BK] halves (k-contiguous; with
//    BK = 64 every load fetches 8 whole 128-byte rows, full cache lines), B
//    as KSUB sub-tiles of [32][BN] halves (n-contiguous, as it lies in
//    memory). The loads are limited by the rate of L2 requests, so whole
//    lines matter: 64-byte rows of A took as many requests as 128-byte ones.
//  * Each tile starts its walk over K at step (tm + tn) mod (number of
//    steps) and wraps around. The tiles of one die that share an A row panel
//    (or a B column panel) then read different K steps of it at any moment
//    instead of all requesting the same lines at once: 1024^3 8.89 -> 8.28
//    us, 2048^3 37.0 -> 33.3 us. With fewer than 8 steps (K < 512: every
//    load is a first touch from HBM) the tiles keep step 0 first, where
//    reading the same lines together shares their latency (256^3 ran 4.16
//    us in step, 4.33 skewed). A tile's K order is fixed by its position, so
//    results do not depend on launch order.
//  * One barrier per step. The fragments of step j + 1 are read from LDS
//    (ds_read_b128 for A, the transposing ds_read_b64_tr_b16 for B) while the
//    matrix ops of step j run from registers, and the loads of step
//    j + STAGES go into the slot that step j occupied, so the barrier is the
//    only wait between the waves.
//  * v_mfma_f32_32x32x16_f16 with the B fragment as the first operand: each
//    lane of a 32 x 32 result holds runs of four consecutive columns of one
//    row of C. Two accumulator sets (even and odd 16-deep halves) keep
//    consecutive matrix ops independent; they are added in the epilogue.
//  * Epilogue: ReLU (or bias + GELU) and the round-to-nearest-even fp16
//    conversion in registers, then 8-byte stores of each lane's four-column
//    runs (the C tile is small; the L2 merges the partial lines).
//
// Requirements (checked on the host): operands as stored (NN), K and N
// multiples of 8, A, B and C 16-byte aligned, in-tile offsets below 2^31.
#pragma once

#include <utility>

#include "common.hpp"

namespace gemm_relu {
namespace small {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int KSUB_ = 2, int STAGES_ = 4>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, KSUB = KSUB_, BK = 32 * KSUB_, STAGES = STAGES_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NW = WAVES_M * WAVES_N, NT = kWave * NW;
    static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // wave sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;              // 32 x 32 blocks per wave
    static constexpr int A_STEP = BM * BK, B_SUB = 32 * BN;       // halves: A per step, B per 32 deep
    static constexpr int SLOT = A_STEP + KSUB * B_SUB;            // halves per ring slot
    static constexpr int A_ROW_BYTES = BK * 2;                    // one A row of a step
    static constexpr int A_ROWS_PER_LOAD = 1024 / A_ROW_BYTES;
    static constexpr int A_LOADS = BM / A_ROWS_PER_LOAD;          // 1 KiB loads per step
    static constexpr int B_LOADS = KSUB * BN / 16;                // 512 / BN k-rows of B each
    static constexpr int LPW = (A_LOADS + B_LOADS) / NW;          // loads per wave per step
    static constexpr int B_LANES_PER_ROW = BN / 8;                // 16-byte chunks per row of B
    static constexpr int NMMA = KSUB * 2 * FM * FN;               // matrix ops per wave per step
    static constexpr int NREAD = KSUB * 2 * (FM + 2 * FN);        // LDS read instructions per step
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave sub-tiles of whole 32 x 32 blocks");
    static_assert(KSUB == 1 || KSUB == 2, "64- or 128-byte A rows");
    static_assert(BM % A_ROWS_PER_LOAD == 0 && BN >= 64 && 512 % BN == 0, "1 KiB loads cover whole rows");
    static_assert((A_LOADS + B_LOADS) % NW == 0, "loads split evenly over the waves");
    static_assert(STAGES == 4 || STAGES == 6 || STAGES == 8, "an even ring of 4 to 8 slots (fragments alternate)");
    static_assert((STAGES - 2) * LPW < 64, "vmcnt range");
    static_assert(STAGES * SLOT * 2 <= 160 * 1024, "LDS");
};

// A step row r (BK halves, 64 or 128 bytes): logical 16-byte chunk c at
// physical chunk c ^ a_swz(r). With 64-byte rows this is the large tile's A
// swizzle (zero bank conflicts measured on this fragment read): 4 rows share
// a 256-byte bank window and each group of 4 rows takes another rotation.
// With 128-byte rows 2 rows share a window, and (r / 2) % 8 gives 16
// consecutive rows read at one logical chunk 16 different 16-byte slots.
template <int BK>
__device__ __forceinline__ int a_swz(int r)
{
    if constexpr (BK == 32) return (r >> 2) & 3;
    else return (r >> 1) & 7;
}

// B sub-tile k-row kr (BN halves): logical chunk c at c ^ b_swz(kr), moving
// 32-byte column pairs by kr % 4 as the large tile's B swizzle does.
__device__ __forceinline__ int b_swz(int kr) { return 2 * (kr & 3); }

template <class T, bool KALIGNED>
__global__ void __launch_bounds__(T::NT, T::NW >= 4 ? 2 : 3) small_kernel(Args p)
{
    constexpr int R = T::STAGES;
    __shared__ __attribute__((aligned(1024))) uint16_t st0[T::SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st1[T::SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st2[T::SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st3[T::SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st4[R > 4 ? T::SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st5[R > 5 ? T::SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st6[R > 6 ? T::SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st7[R > 7 ? T::SLOT : 8];
    auto slot = [&]<int S>() -> uint16_t* {
        static_assert(S >= 0 && S < R, "ring slot");
        if constexpr (S == 0) return st0;
        else if constexpr (S == 1) return st1;
        else if constexpr (S == 2) return st2;
        else if constexpr (S == 3) return st3;
        else if constexpr (S == 4) return st4;
        else if constexpr (S == 5) return st5;
        else if constexpr (S == 6) return st6;
        else return st7;
    };

    GR_STAMP_DECL;
    GR_STAMP(0);
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int M = p.M, N = p.N, K = p.K;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const int nk = (K + T::BK - 1) / T::BK;
    const int kskew = nk >= 8 ? (tm + tn) % nk : 0;  // this tile's first K step

    // ---- this wave's loads: global byte offsets (relative to A + m0*K + k0
    // and B + k0*N), LDS destinations (halves within a slot), K-tail chunks ----
    uint32_t goff[T::LPW];
    int ldst[T::LPW];
    int kcol[T::LPW];  // first k of the lane's chunk within the step (A only)
    bool is_a[T::LPW];
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
        const int gi = wave * T::LPW + i;
        if (gi < T::A_LOADS) {
            // whole rows of the step: A_ROWS_PER_LOAD rows of BK halves
            constexpr int LPR = T::BK / 8;  // lanes per row
            const int row = gi * T::A_ROWS_PER_LOAD + lane / LPR;
            const int c = (lane % LPR) ^ a_swz<T::BK>(row);
            is_a[i] = true;
            kcol[i] = c * 8;
            goff[i] = (m0 + row < M) ? (uint32_t)(row * K + c * 8) * 2u : kOOB;
            ldst[i] = gi * 512;
        } else {
            const int gj = gi - T::A_LOADS;
            const int s = gj / (T::BN / 16), rb = gj % (T::BN / 16);
            const int kr = rb * (512 / T::BN) + lane / T::B_LANES_PER_ROW;
            const int c = (lane % T::B_LANES_PER_ROW) ^ b_swz(kr);
            is_a[i] = false;
            kcol[i] = 0;
            // rows past K are cut off by the descriptor's byte count
            goff[i] = (n0 + c * 8 < N) ? (uint32_t)((s * 32 + kr) * N + n0 + c * 8) * 2u : kOOB;
            ldst[i] = T::A_STEP + s * T::B_SUB + rb * 512;
        }
    }

    // Descriptors of the steps. Step kt reads the K columns [k0, k0 + BK),
    // k0 = ((kt + kskew) % nk) * BK; steps past the end of K get empty
    // descriptors (every lane out of range: zeros). A cursor walks the steps
    // with a few scalar additions, and the next step's descriptors are made
    // a piece at a time between the matrix ops (built from kt at once, they
    // were a run of some 60 scalar instructions in front of the barrier).
    struct Rsrc {
        __amdgpu_buffer_rsrc_t a, b;
        int kleft;  // K columns from the step's first to the end of K (0 past the end)
    };
    struct Cursor {
        int kt, s;            // the step, and its place in the walk: k0 = s * BK
        uint64_t aoff, boff;  // byte offsets of column k0 from column 0
    };
    const char* const abase0 = reinterpret_cast<const char*>(p.A + (int64_t)m0 * K);
    const char* const bbase0 = reinterpret_cast<const char*>(p.B);
    const uint64_t arem0 = (uint64_t)(M - m0) * K * 2, brem0 = (uint64_t)K * N * 2;
    const uint32_t astep = T::BK * 2, bstep = (uint32_t)(T::BK * 2) * (uint32_t)N;  // N <= 2^24: at most 2^31
    auto cursor_at = [&](int kt) -> Cursor {
        const int s = nk > 0 ? (kt + kskew) % nk : 0;
        return {kt, s, (uint64_t)s * astep, (uint64_t)s * bstep};
    };
    auto advance = [&](Cursor& c) {
        c.kt += 1;
        const bool wrap = c.s + 1 == nk;
        c.s = wrap ? 0 : c.s + 1;
        c.aoff = wrap ? 0 : c.aoff + astep;
        c.boff = wrap ? 0 : c.boff + bstep;
    };
    // record count: the bytes left, at most 2^31, in 32-bit scalar operations
    // (the compiler would otherwise fold the test into a 64-bit comparison,
    // which goes through vector registers)
    auto records = [](uint64_t bytes, bool live) -> int {
        uint32_t hi = (uint32_t)(bytes >> 32);
        const uint32_t lo = (uint32_t)bytes;
        asm("" : "+s"(hi));
        const uint32_t n = (hi | (lo >> 31)) != 0 ? (uint32_t)kMaxRecords : lo;
        return live ? (int)n : 0;
    };
    auto desc_a = [&](const Cursor& c) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(abase0 + c.aoff), (short)0,
                                                 records(arem0 - c.aoff, c.kt < nk), kRsrcWord3);
    };
    auto desc_b = [&](const Cursor& c) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(bbase0 + c.boff), (short)0,
                                                 records(brem0 - c.boff, c.kt < nk), kRsrcWord3);
    };
    auto kleft = [&](const Cursor& c) { return c.kt < nk ? K - c.s * T::BK : 0; };
    auto descriptors = [&](const Cursor& c) -> Rsrc { return {desc_a(c), desc_b(c), kleft(c)}; };
    // this wave's load i of the step of r into ring slot S
    auto load_one = [&]<int S>(int i, const Rsrc& r) {
        uint16_t* dst = slot.template operator()<S>() + ldst[i];
        if (is_a[i]) {
            const __amdgpu_buffer_rsrc_t ra = r.a;
            uint32_t off = goff[i];
            if constexpr (!KALIGNED) off = (kcol[i] < r.kleft) ? off : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (GR_LDS void*)dst, 16, (int)off, 0, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rb = r.b;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (GR_LDS void*)dst, 16, (int)goff[i], 0, 0, 0);
        }
    };

    // ---- fragment read addresses (bytes within a slot) ----
    // A block i, 16-deep part sh = 2s + h of the step: row wm*TM + 32i +
    // lane%32, logical chunk 2 sh + lane/32
    const int arow = wm * T::TM + lane % 32;
    uint32_t a_rd[2 * T::KSUB];
#pragma unroll
    for (int sh = 0; sh < 2 * T::KSUB; ++sh)
        a_rd[sh] = arow * T::A_ROW_BYTES + (((2 * sh + lane / 32) ^ a_swz<T::BK>(lane % 32)) * 16);
    // B block j, half h, read t: the 16-lane group g reads k-row 16h + 8(g/2)
    // + 4t + (lane%16)/4 and columns wn*TN + 32j + 16(g%2) + 4(lane%4) .. +3;
    // after the transpose the lane holds column wn*TN + 32j + lane%32 at four
    // consecutive k.
    const int g = lane / 16, q16 = lane % 16;
    uint32_t b_rd[2][2][T::FN];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const int kr = 16 * h + 8 * (g / 2) + 4 * t + q16 / 4;
                const int col = wn * T::TN + 32 * j + 16 * (g % 2) + 4 * (q16 % 4);
                b_rd[h][t][j] = kr * (T::BN * 2) + (((col / 8) ^ b_swz(kr)) * 16) + 8 * ((col / 4) % 2);
            }

    // the fragments of one step: [sub-tile][half][block]
    struct Frag {
        f16x8 a[T::KSUB][2][T::FM];
        f16x8 b[T::KSUB][2][T::FN];
    };
    auto tr_read = [](const char* base) -> i16x4 {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS i16x4*)(base));
    };
    // read instruction q (0 .. NREAD-1) of the step in slot S into f: per
    // (sub-tile, half), FM A reads then FN pairs of B reads
    auto read_one = [&]<int S>(int q, Frag& f) {
        constexpr int PER = T::FM + 2 * T::FN;
        const int sh = q / PER, r = q % PER;
        const int s = sh / 2, h = sh % 2;
        const char* sa = reinterpret_cast<const char*>(slot.template operator()<S>());
        const char* sb = reinterpret_cast<const char*>(slot.template operator()<S>()) + (T::A_STEP + s * T::B_SUB) * 2;
        if (r < T::FM) {
            f.a[s][h][r] = *reinterpret_cast<const f16x8*>(sa + a_rd[2 * s + h] + r * 32 * T::A_ROW_BYTES);
        } else {
            const int j = (r - T::FM) / 2, t = (r - T::FM) % 2;
            const i16x4 v = tr_read(sb + b_rd[h][t][j]);
            // halves 0-3 of the fragment from read t = 0, 4-7 from t = 1
            i16x8 w = __builtin_bit_cast(i16x8, f.b[s][h][j]);
            if (t == 0) {
                w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
            } else {
                w[4] = v[0]; w[5] = v[1]; w[6] = v[2]; w[7] = v[3];
            }
            f.b[s][h][j] = __builtin_bit_cast(f16x8, w);
        }
    };

    f32x16 acc[2][T::FM][T::FN];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[e][i][j][r] = 0.0f;

    // matrix op u of a step: (sub-tile, half) = u / (FM FN), block (i, j);
    // halves alternate between the two accumulator sets
    auto mma_one = [&](const Frag& f, int u) {
        const int sh = u / (T::FM * T::FN), ij = u % (T::FM * T::FN);
        const int s = sh / 2, h = sh % 2, i = ij / T::FN, j = ij % T::FN;
        acc[h][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[s][h][j], f.a[s][h][i], acc[h][i][j], 0, 0, 0);
    };

    // wait until this wave's loads older than the newest N have landed and
    // its LDS reads are done, then meet the other waves
    auto sync = [&]<int N>() {
        static_assert(N >= 0 && N < 64, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Region j (slot S = j % R): wait for step j+1 (steps up to j+R-1 may
    // still be in flight), barrier, then the matrix ops of step j (fragments
    // x) with the loads of step j+R (into slot S, which every wave finished
    // reading before the barrier) and the fragment reads of step j+1 (into
    // y) spread between them. The ring runs nkr = nk rounded up to a
    // multiple of R steps; the extra steps multiply zero tiles.
    const int nkr = (nk + R - 1) / R * R;
    constexpr int NMEM = T::LPW + T::NREAD;
    // after which matrix ops the cursor moves on and the next descriptors are made
    constexpr int kAdvU = T::NMMA > 1 ? 1 : 0, kDescAU = T::NMMA > 2 ? 2 : T::NMMA - 1,
                  kDescBU = T::NMMA > 3 ? 3 : T::NMMA - 1;
    Cursor cur = cursor_at(0);  // the next step to load
    Rsrc r, rn;                 // its descriptors, and the following step's
    auto region = [&]<int S>(Frag& x, Frag& y) {
        constexpr int S1 = (S + 1) % R;
        const Rsrc rs = r;  // step j + R
        sync.template operator()<(R - 2) * T::LPW>();
        int m = 0;
#pragma unroll
        for (int u = 0; u < T::NMMA; ++u) {
            mma_one(x, u);
            // this op's share of the memory items: loads first, then reads
            const int m_end = (NMEM * (u + 1)) / T::NMMA;
#pragma unroll
            for (; m < m_end; ++m) {
                if (m < T::LPW) load_one.template operator()<S>(m, rs);
                else read_one.template operator()<S1>(m - T::LPW, y);
            }
            if (u == kAdvU) advance(cur);
            if (u == kDescAU) rn.a = desc_a(cur);
            if (u == kDescBU) {
                rn.b = desc_b(cur);
                rn.kleft = kleft(cur);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        r = rn;
    };

    Frag x, y;
    if (nkr > 0) {
        // prologue: steps 0 .. R-1 in flight, then wait for step 0 and read it
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (
                [&] {
                    const Rsrc r0 = descriptors(cur);
#pragma unroll
                    for (int i = 0; i < T::LPW; ++i) load_one.template operator()<I>(i, r0);
                    advance(cur);
                }(),
                ...);
        }(std::make_integer_sequence<int, R>{});
        r = descriptors(cur);
        sync.template operator()<(R - 1) * T::LPW>();
        GR_STAMP(1);
#pragma unroll
        for (int q = 0; q < T::NREAD; ++q) read_one.template operator()<0>(q, x);
    }
    // R regions per pass, fragments alternating between x and y
    for (int j = 0; j < nkr; j += R) {
        [&]<int... S>(std::integer_sequence<int, S...>) {
            ((S % 2 == 0 ? region.template operator()<S>(x, y) : region.template operator()<S>(y, x)), ...);
        }(std::make_integer_sequence<int, R>{});
    }
    // the zero-filling loads past the end must land before the waves exit
    __builtin_amdgcn_s_waitcnt(0);
    GR_STAMP(2);

    // ---- epilogue: lane holds, for rows 32i + lane%32 of the wave tile, the
    // columns 32j + 8q + 4(lane/32) + 0..3 in acc[.][i][j][4q .. 4q+3] ----
    with_epilogue(p, [&]<int ACT>() {
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * T::TN + 32 * j + 8 * q + 4 * (lane / 32);
                const f32x4 bias = (ACT == kActBiasGelu) ? bias4(p, n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < T::FM; ++i) {
                    const int m = m0 + wm * T::TM + 32 * i + lane % 32;
                    u32x2 w;
                    w[0] = epi_pack2b<ACT>(acc[0][i][j][4 * q + 0] + acc[1][i][j][4 * q + 0],
                                           acc[0][i][j][4 * q + 1] + acc[1][i][j][4 * q + 1], bias[0], bias[1]);
                    w[1] = epi_pack2b<ACT>(acc[0][i][j][4 * q + 2] + acc[1][i][j][4 * q + 2],
                                           acc[0][i][j][4 * q + 3] + acc[1][i][j][4 * q + 3], bias[2], bias[3]);
                    if (m < M && n < N) *reinterpret_cast<u32x2*>(p.C + (int64_t)m * N + n) = w;
                }
            }
        }
    });
    GR_STAMP_FLUSH(p);
}

}  // namespace small
}  // namespace gemm_relu

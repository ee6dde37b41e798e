// Pipelined kernel for large tiles: the hot path at big problem sizes.
//
// Same computation as the TileLang GEMM + ReLU example ("Writing
// high-performance kernels in TileLang", section "Escribamos un GEMM"):
// a BM x BN tile of C per workgroup, K walked in BK-wide steps staged through
// shared memory, fp32 accumulators in registers, max(x, 0), fp16 store. The
// gfx950 design:
//
//  * Direct-to-LDS loads. Each `buffer_load_dwordx4 ... lds` moves 1 KiB (64
//    lanes x 16 B) from global memory straight into LDS without passing
//    through registers. A lane whose element lies outside the matrix is given
//    an offset past the buffer's end and the hardware writes zeros: that is
//    the masking of ragged edge tiles (M, N and the K tail).
//  * A four-slot LDS ring of BK = 32 steps (4 x 32 KiB at 256 x 256): while
//    step k is multiplied, steps k+1 and k+2 are in flight and step k+3 is
//    issued. Each slot is its own LDS array, so the compiler can tell the
//    slots apart and never drains the whole ring.
//  * One barrier per step. Between two barriers a wave runs 32 matrix
//    operations: the second half of one step and the first half of the next.
//    The first two of them do not depend on the barrier and are issued before
//    it, so the matrix cores have work while the waves meet. The loads of a
//    later step are spread evenly over the region and the fragment reads of
//    the next two halves are issued one slot at a time between the matrix
//    operations, in an order fixed in the source: a burst of loads would
//    hold the matrix operations queued behind it until the address unit had
//    taken them all.
//  * Tile products on v_mfma_f32_32x32x16_f16 (one 64-lane wave per TM x TN
//    sub-tile). The B fragment is the first operand, so each lane of the
//    32x32 result holds runs of four consecutive columns of one row of C.
//  * A is stored k-contiguous ([BM][32]) and read with ds_read_b128. B is
//    stored as it lies in memory, n-contiguous ([32][BN]), and read with the
//    gfx950 transposing LDS load ds_read_b64_tr_b16, which hands each lane
//    four k-values of one column: no register transpose.
//  * Transposed operands (the transpose_A / transpose_B of the pages' tile
//    product): every operand tile keeps the layout it has in memory. A
//    stored K x M is staged m-contiguous ([32][BM]) and read with the
//    transposing load; B stored N x K is staged k-contiguous ([BN][32]) and
//    read with ds_read_b128. Fragments come out in the same lanes either way,
//    so the matrix ops and the epilogue do not change.
//  * XOR swizzles of the 16-byte chunk index (applied when choosing which
//    global chunk each lane fetches) spread the fragment reads over the LDS
//    banks; the direct loads themselves write 1 KiB linearly.
//  * When K is a multiple of 32 (KALIGNED) no step is partial: the loads carry
//    no per-lane K test and each step only moves two buffer descriptors.
//  * Epilogue: the fp32 accumulators go through v_cvt_pk_f16_f32 (round to
//    nearest even) and a packed max with zero (ReLU) into the now idle LDS
//    ring, which holds the whole 256 x 256 fp16 tile; then every lane stores
//    16 consecutive bytes of a row, so each store instruction writes two full
//    512-byte rows of C. Epilogue arithmetic runs at a quarter of the issue
//    rate (64 lanes on 16-lane SIMDs) and all CUs reach it at once, so it is
//    kept to two instructions per pair of outputs.
//
// Requirements (checked on the host): the leading dimension of each operand
// (K or M for A, N or K for B) and N are multiples of 8, A, B and C are
// 16-byte aligned, and every in-tile offset (BM * K, 32 * M, 32 * N, BN * K
// halves) stays below 2^30.
#pragma once

#include <utility>

#include "common.hpp"

namespace gemm_relu {
namespace pipelined {

// tiles one launch places one per compute unit (256 CUs)
constexpr int kSkewTilesOneRound = 256;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_ = 4, bool APAIR_ = false>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, STAGES = STAGES_;
    // A stored M x K is loaded two steps at a time (128 bytes of each row:
    // whole cache lines) into one of two pair arrays; steps 2p and 2p+1
    // share it.
    static constexpr bool APAIR = APAIR_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NW = WAVES_M * WAVES_N, NT = kWave * NW;
    static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // wave sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;              // 32x32 MFMA blocks
    static constexpr int A_HALVES = BM * BK, B_HALVES = BK * BN;  // per stage
    static constexpr int STAGE_BYTES = (A_HALVES + B_HALVES) * 2;
    static constexpr int A_LOADS = A_HALVES * 2 / 1024;            // 1 KiB loads per stage
    static constexpr int B_LOADS = B_HALVES * 2 / 1024;
    static constexpr int A_LOADS_W = A_LOADS / NW, B_LOADS_W = B_LOADS / NW;
    static constexpr int LPT = A_LOADS_W + B_LOADS_W;              // loads per wave per step
    static constexpr int B_ROW_BYTES = BN * 2;
    static constexpr int NMMA = FM * FN;                           // matrix ops per half-step
    static constexpr int NSLOT = FM + FN;                          // fragment-read slots per half-step
    // epilogue: the fp16 C tile (BN * 2 bytes per row) goes through the first
    // slots of the ring, C_ROWS_PER_STAGE rows per slot: the largest
    // multiple of 32 rows that fits in a slot, rounded down to a power of two
    // so that blocks of 32 rows never straddle two slots
    static constexpr int C_ROWS_FIT = STAGE_BYTES / (BN * 2);
    static constexpr int C_ROWS_PER_STAGE = C_ROWS_FIT >= 128 ? 128 : C_ROWS_FIT >= 64 ? 64 : 32;
    static constexpr int C_ROWS_PER_PASS = NT / (BN / 8);  // rows stored per pass (16 B per lane)
    static_assert(A_LOADS % NW == 0 && B_LOADS % NW == 0, "loads must split evenly over waves");
    static_assert(TM % 32 == 0 && TN % 128 == 0, "wave sub-tile: 32-row blocks, 128-column units");
    static_assert(2 * LPT < 64, "vmcnt range");
    static_assert(STAGES >= 3 && STAGES <= 8, "ring of 3 to 8 slots (one LDS array each)");
    static_assert((STAGES - 2) * LPT < 64, "vmcnt range");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
    static_assert(C_ROWS_FIT >= 32 && BM <= STAGES * C_ROWS_PER_STAGE, "the C tile must fit in the ring");
    static_assert(C_ROWS_PER_STAGE % C_ROWS_PER_PASS == 0, "a store pass stays in one slot");
    static_assert(BN == 256, "the epilogue maps 32 lanes x 16 B onto one row of C");
    static constexpr int AP_LOADS_W = APAIR ? BM * 64 * 2 / 1024 / NW : 0;  // 1 KiB loads per wave per pair
    static_assert(!APAIR || (STAGES == 4 && (BM / NW) % 16 == 0 && BM <= 256),
                  "paired A steps: a four-slot ring, 16 rows or a multiple per wave");
};

// A: row r of a stage holds 32 halves = four 16-byte chunks; logical chunk c
// sits at physical chunk c ^ a_swz(r), with a_swz(r) = (r / 4) % 4. Four
// consecutive rows fill one 256-byte bank window, and each of the next three
// groups of four takes another rotation of the chunks, so sixteen consecutive
// rows read at one logical chunk touch every bank once. Measured with the
// LDS bank-conflict counter on the fragment read below (32 rows, two logical
// chunks per lane pair): zero conflicts; an XOR with row bits 1 and 3, which
// spreads 16 rows just as well on paper, left a third of the read's LDS
// cycles as conflicts, as did bits 1-2, so gfx950 does not serve a 16-byte
// read in groups of 16 consecutive lanes.
__device__ __forceinline__ int a_swz(int r) { return (r >> 2) & 3; }

// A with paired steps: row r holds 64 halves = eight 16-byte chunks (two
// steps); logical chunk c sits at physical chunk c ^ ap_swz(r). Two rows fill
// a 256-byte bank window, and (r / 2) % 8 gives the rows of each parity in
// any 16 consecutive ones eight different chunks, so a fragment read of 16
// rows at one logical chunk touches every bank once.
__device__ __forceinline__ int ap_swz(int r) { return (r >> 1) & 7; }

// B: row kr of a stage holds BN halves; logical chunk c sits at physical chunk
// c ^ b_swz(kr). A transposing read touches four consecutive rows (kr % 4 =
// 0..3) at one 32-byte column pair; XOR-ing the pair index with kr % 4 spreads
// them over four pairs.
__device__ __forceinline__ int b_swz(int kr) { return 2 * (kr & 3); }

// Transposed A, staged m-contiguous: row kr of a stage holds BM halves. Its
// transposing reads take 32-byte column pairs p and p + 1 (two 16-lane groups)
// from four consecutive rows, so the XOR moves whole pairs by an even amount:
// with rows of 256 bytes or more, 2 (kr % 4) pairs, which puts the eight
// (row, pair) reads of 32 lanes on eight pairs of one 256-byte bank window;
// with 128-byte rows (BM = 64), where rows kr and kr + 2 share a window, 2
// pairs for kr / 2 odd.
template <int BM>
__device__ __forceinline__ int at_swz(int kr)
{
    if constexpr (BM >= 128) return 4 * (kr & 3);
    else return 4 * ((kr >> 1) & 1);
}

// Epilogue C tile in LDS: row r (BN halves = 32 chunks of 16 B), logical chunk
// c at physical chunk c ^ (r % 32), so the 32 rows that one store of the
// accumulator layout touches land on 32 different chunks.
__device__ __forceinline__ int c_swz(int r) { return r & 31; }

// Which memory items follow the matrix op at each position of a region of
// 2 * NMMA ops (positions 0..NMMA-1 use fragments y, the rest x). Positions
// up to PRE hold the barrier. After them:
//  * the NSLOT read slots of x, one per position, all before block x starts;
//  * the NSLOT read slots of y, one per position from the start of block x
//    (after the last op that reads y);
//  * the LPT loads spread evenly over every position after PRE, at most one
//    per position (a position may hold a load and a read slot).
template <int NMMA, int NSLOT, int LPT, int PRE>
struct RegionPlan {
    static constexpr int kPositions = 2 * NMMA;
    int load[kPositions];   // load index or -1
    int readx[kPositions];  // x read slot or -1
    int ready[kPositions];  // y read slot or -1
    constexpr RegionPlan() : load{}, readx{}, ready{}
    {
        for (int q = 0; q < kPositions; ++q) load[q] = readx[q] = ready[q] = -1;
        for (int i = 0; i < NSLOT; ++i) {
            readx[PRE + 1 + i] = i;
            ready[NMMA + i] = i;
        }
        const int span = kPositions - PRE - 1;
        for (int v = 0; v < LPT; ++v) load[PRE + 1 + (v * span) / LPT] = v;
    }
    static constexpr bool fits() { return PRE + 1 + NSLOT <= NMMA && NSLOT <= NMMA && LPT <= kPositions - PRE - 1; }
};

// COUNT loads spread evenly over the positions [FIRST, END) of a region of
// 2 NMMA matrix ops: count[q] of them at position q, numbered from first[q]
// (several to a position when there are more loads than positions).
template <int NMMA, int FIRST, int END, int COUNT>
struct LoadSpread {
    static_assert(0 <= FIRST && FIRST < END && END <= 2 * NMMA, "positions inside the region");
    int first[2 * NMMA];
    int count[2 * NMMA];
    constexpr LoadSpread() : first{}, count{}
    {
        for (int q = 0; q < 2 * NMMA; ++q) first[q] = count[q] = 0;
        for (int v = 0; v < COUNT; ++v) {
            const int q = FIRST + (v * (END - FIRST)) / COUNT;
            if (count[q] == 0) first[q] = v;
            ++count[q];
        }
    }
};

template <class T, bool KALIGNED, bool TA = false, bool TB = false>
__global__ void __launch_bounds__(T::NT, 1) pipelined_kernel(Args p)
{
    // One LDS array per stage (A tile, then B tile): the compiler tracks
    // direct-to-LDS writes per array, so distinct arrays keep the reads of
    // one stage from waiting on the loads into another.
    // (Two slots in one array would make the reads of either wait for the
    // loads into both.) Arrays past the ring's last slot are never referenced
    // and take no LDS.
    // Paired A (AP): the A pairs live in two arrays of their own and the B
    // steps in four, so that every fragment read and every load names its
    // array at compile time (a pointer chosen between two arrays at run time
    // makes the compiler wait for every load in flight before each read).
    constexpr bool AP = T::APAIR && !TA;
    constexpr int SLOT = AP ? 8 : T::A_HALVES + T::B_HALVES;
    __shared__ __attribute__((aligned(1024))) uint16_t pa0[AP ? T::BM * 64 : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t pa1[AP ? T::BM * 64 : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t sb0[AP ? T::B_HALVES : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t sb1[AP ? T::B_HALVES : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t sb2[AP ? T::B_HALVES : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t sb3[AP ? T::B_HALVES : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st0[SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st1[SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st2[SLOT];
    __shared__ __attribute__((aligned(1024))) uint16_t st3[T::STAGES > 3 ? SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st4[T::STAGES > 4 ? SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st5[T::STAGES > 5 ? SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st6[T::STAGES > 6 ? SLOT : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t st7[T::STAGES > 7 ? SLOT : 8];
    auto stage_a = [&]<int S>() -> uint16_t* {
        static_assert(S >= 0 && S < T::STAGES, "ring slot");
        if constexpr (S == 0) return st0;
        else if constexpr (S == 1) return st1;
        else if constexpr (S == 2) return st2;
        else if constexpr (S == 3) return st3;
        else if constexpr (S == 4) return st4;
        else if constexpr (S == 5) return st5;
        else if constexpr (S == 6) return st6;
        else return st7;
    };
    auto stage_b = [&]<int S>() -> uint16_t* {
        if constexpr (AP) {
            static_assert(S >= 0 && S < 4, "ring slot");
            if constexpr (S == 0) return sb0;
            else if constexpr (S == 1) return sb1;
            else if constexpr (S == 2) return sb2;
            else return sb3;
        } else {
            return stage_a.template operator()<S>() + T::A_HALVES;
        }
    };
    auto pair_a = [&]<int PS>() -> uint16_t* {
        if constexpr (PS == 0) return pa0;
        else return pa1;
    };

    static_assert(!TA || (T::BM >= 64 && 512 % T::BM == 0), "a transposed A tile row is 64 to 512 halves");
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
    // This tile's first K step (the walk wraps around): tiles of a die that
    // share an A row panel or a B column panel then read different steps of
    // it at any moment instead of requesting the same lines at once.
    // 64- and 128-row tiles skew over the whole K range (2048^3 33.3 -> 31.2
    // us). 256 x 256 tiles skew by at most 7 steps, and only when there are
    // more tiles than CUs (8192 x 8192 x 1024: 141.2 -> 134.0 us): with one
    // tile per CU, as at 4096^3, the dies' tiles walk K in step and share
    // what each die fetches, and a skew measured no better. Below 8 steps
    // every load is a first touch from HBM, where reading the same lines
    // together shares their latency.
    int kskew = 0;
    if (nk >= 8) {
        if constexpr (T::BM == 256 && T::BN == 256)
            kskew = p.tiles_m * p.tiles_n > kSkewTilesOneRound ? ((tm + tn) % 8) % nk : 0;
        else
            kskew = (tm + tn) % nk;
    }
    // paired A steps: a pair starts on an even step of the walk and never
    // wraps inside it
    if constexpr (AP) kskew = nk % 2 == 0 ? (kskew & ~1) : 0;

    // ---- per-lane global offsets of this wave's direct loads (bytes, relative
    // to the step's descriptor base: A + m0*K + k0 and B + k0*N) ----
    // (A stored K x M: relative to A + k0*M; B stored N x K: to B + n0*K + k0)
    uint32_t a_off[T::A_LOADS_W];
    int a_kc[T::A_LOADS_W];  // logical k-chunk of the lane, for the K tail
#pragma unroll
    for (int i = 0; i < T::A_LOADS_W; ++i) {
        const int gi = wave * T::A_LOADS_W + i;
        if constexpr (!TA) {
            const int row = gi * 16 + lane / 4;
            const int c = (lane % 4) ^ a_swz(row);
            a_kc[i] = c;
            a_off[i] = (m0 + row < M) ? (uint32_t)(row * K + c * 8) * 2u : kOOB;
        } else {
            // one 1 KiB load covers 512 / BM k-rows of BM halves
            constexpr int LPR = T::BM / 8;
            const int kr = gi * (64 / LPR) + lane / LPR;
            const int c = (lane % LPR) ^ at_swz<T::BM>(kr);
            a_kc[i] = 0;
            // rows past K are cut off by the descriptor's byte count
            a_off[i] = (m0 + c * 8 < M) ? (uint32_t)(kr * M + m0 + c * 8) * 2u : kOOB;
        }
    }
    // paired A (AP): load v of a wave covers rows 64 wave + 8 v .. + 7, 128
    // bytes each (16 bytes per lane), of the pair's two steps. The lane's
    // chunk depends on v only through v % 2 (the swizzle repeats every 16
    // rows), so two offsets serve all loads; rows past M lie beyond the
    // descriptor's byte count and read as zeros.
    uint32_t ap_off[2];
    int ap_kc[2];  // logical k-chunk (0..7) of the lane within the pair
    if constexpr (AP) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int row = wave * (T::BM / T::NW) + 8 * e + lane / 8;
            const int c = (lane % 8) ^ ap_swz(row);
            ap_kc[e] = c;
            ap_off[e] = (uint32_t)(row * K + c * 8) * 2u;
        }
    }
    uint32_t b_off[T::B_LOADS_W];
    int b_kc[T::B_LOADS_W];
#pragma unroll
    for (int i = 0; i < T::B_LOADS_W; ++i) {
        const int gi = wave * T::B_LOADS_W + i;
        if constexpr (!TB) {
            const int kr = gi * 2 + lane / 32;
            const int c = (lane % 32) ^ b_swz(kr);
            b_kc[i] = 0;
            // rows past K are cut off by the descriptor's byte count
            b_off[i] = (n0 + c * 8 < N) ? (uint32_t)(kr * N + n0 + c * 8) * 2u : kOOB;
        } else {
            const int row = gi * 16 + lane / 4;
            const int c = (lane % 4) ^ a_swz(row);
            b_kc[i] = c;
            b_off[i] = (n0 + row < N) ? (uint32_t)(row * K + c * 8) * 2u : kOOB;
        }
    }

    // Buffer descriptors of the steps. Step kt reads the K columns [k0, k0 +
    // BK), k0 = ((kt + kskew) % nk) * BK; steps past the end of K get empty
    // descriptors: every lane is out of range and the stage fills with zeros.
    // A cursor walks the steps with a few scalar additions (recomputing a
    // step's descriptors from kt took a modulo and 64-bit products, some 60
    // scalar instructions in a row that held up the matrix ops behind them).
    struct Rsrc {
        __amdgpu_buffer_rsrc_t a, b;
        int kleft;  // K columns from the step's first to the end of K (0 past the end)
    };
    struct Cursor {
        int kt, s;            // the step, and its place in the walk: k0 = s * BK
        uint64_t aoff, boff;  // byte offsets of column k0 from column 0
    };
    const char* const abase0 = reinterpret_cast<const char*>(TA ? p.A : p.A + (int64_t)m0 * K);
    const char* const bbase0 = reinterpret_cast<const char*>(TB ? p.B + (int64_t)n0 * K : p.B);
    const uint64_t arem0 = TA ? (uint64_t)K * M * 2 : (uint64_t)(M - m0) * K * 2;
    const uint64_t brem0 = TB ? (uint64_t)(N - n0) * K * 2 : (uint64_t)K * N * 2;
    // bytes per step (below 2^31: 32 M and 32 N halves are below 2^30)
    const uint32_t astep = TA ? (uint32_t)(T::BK * 2) * (uint32_t)M : (uint32_t)(T::BK * 2);
    const uint32_t bstep = TB ? (uint32_t)(T::BK * 2) : (uint32_t)(T::BK * 2) * (uint32_t)N;
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
    // the descriptor's record count: the bytes left, at most kMaxRecords
    // (2^31), in 32-bit scalar operations: the compiler would otherwise fold
    // the test into a 64-bit comparison, which goes through vector registers
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
    auto descriptors = [&](const Cursor& c) -> Rsrc {
        return {desc_a(c), desc_b(c), c.kt < nk ? K - c.s * T::BK : 0};
    };
    // Load number i (A loads first, then B loads) of the step of r into stage S.
    // (The descriptor is copied into a local first: handing the builtin a
    // member of a reference keeps the host side from emitting the kernel.)
    auto load_one = [&]<int S>(int i, const Rsrc& r) {
        uint16_t* sb = stage_b.template operator()<S>();
        if (i < T::A_LOADS_W) {
            uint16_t* sa = nullptr;
            if constexpr (!AP) sa = stage_a.template operator()<S>();
            const __amdgpu_buffer_rsrc_t ra = r.a;
            uint32_t off = a_off[i];
            // a k-contiguous tile masks the K tail per lane
            if constexpr (!KALIGNED && !TA) off = (a_kc[i] * 8 < r.kleft) ? off : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (GR_LDS void*)(sa + (wave * T::A_LOADS_W + i) * 512), 16, (int)off, 0, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rb = r.b;
            const int j = i - T::A_LOADS_W;
            uint32_t off = b_off[j];
            if constexpr (!KALIGNED && TB) off = (b_kc[j] * 8 < r.kleft) ? off : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (GR_LDS void*)(sb + (wave * T::B_LOADS_W + j) * 512), 16, (int)off, 0, 0, 0);
        }
    };

    // Paired A: load v of the pair whose first step is that of r into pair
    // array PS (rows of 64 halves).
    auto load_pair = [&]<int PS>(int v, const Rsrc& r) {
        const __amdgpu_buffer_rsrc_t ra = r.a;
        uint32_t off = ap_off[v % 2] + (uint32_t)(32 * (v / 2)) * (uint32_t)K;  // 16 (v / 2) rows further
        if constexpr (!KALIGNED) off = (ap_kc[v % 2] * 8 < r.kleft) ? off : kOOB;
        const int row0 = wave * (T::BM / T::NW) + 8 * v;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (GR_LDS void*)(pair_a.template operator()<PS>() + row0 * 64), 16, (int)off, 0, 0, 0);
    };
    // B load j of the step of r into stage S
    auto load_b = [&]<int S>(int j, const Rsrc& r) {
        load_one.template operator()<S>(T::A_LOADS_W + j, r);
    };

    // ---- per-lane LDS byte offsets of the fragment reads ----
    // Paired A, step SP (0, 1) of the pair, half h: row wm*TM + 32i + lane%32
    // of the pair array, logical chunk 4 SP + 2h + lane/32. The chunk of the
    // second step differs from the first's in bit 2 only, so its byte offset
    // is the first's with bit 6 flipped.
    uint32_t ap_rd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        ap_rd[h] = (wm * T::TM + lane % 32) * 128 + (((2 * h + lane / 32) ^ ap_swz(lane % 32)) * 16);
    // A block i, half h of a step: row wm*TM + 32i + lane%32, chunk 2h + lane/32.
    const int ar = wm * T::TM + lane % 32;
    uint32_t a_rd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) a_rd[h] = ar * 64 + (((2 * h + lane / 32) ^ a_swz(lane % 32)) * 16);
    // Transposed A (m-contiguous [32][BM]) block i: the 16-lane group g reads
    // rows 8*(g/2) + 4*t + (lane%16)/4 and columns wm*TM + 32i + 16*(g%2) +
    // 4*(lane%4) .. +3, so the lane receives column wm*TM + 32i + lane%32: the
    // same rows of C as the k-contiguous read.
    uint32_t at_rd[T::FM];
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int kr = 8 * ((lane / 16) / 2) + (lane % 16) / 4;
        const int col = wm * T::TM + 32 * i + 16 * ((lane / 16) % 2) + 4 * (lane % 4);
        at_rd[i] = kr * (T::BM * 2) + (((col / 8) ^ at_swz<T::BM>(kr)) * 16) + 8 * ((col / 4) % 2);
    }
    // B block j: the 16-lane group g reads rows 8*(g/2) + 4*t + (lane%16)/4
    // (t = 0, 1 for the two transposing reads) and columns
    //   wn*TN + 128*(j/4) + 16*(j%4) + 64*(g%2) + 4*(lane%4) .. +3,
    // so result row d of the 32x32 block is column 16*(j%4) + 64*(d/16) + d%16
    // of the 128-column unit.
    const int g = lane / 16, q16 = lane % 16;
    uint32_t b_rd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kr = 8 * (g / 2) + q16 / 4;
        const int col = wn * T::TN + 16 * j + 64 * (g % 2) + 4 * (q16 % 4);
        const int c = col / 8;
        b_rd[j] = kr * T::B_ROW_BYTES + ((c ^ b_swz(kr)) * 16) + 8 * ((col / 4) % 2);
    }
    // Transposed B (k-contiguous [BN][32]) block j, half h: the lane reads
    // row wn*TN + 128*(j/4) + 16*(j%4) + 64*(d/16) + d%16 (d = lane % 32) at
    // chunk 2h + lane/32 -- the columns the transposing read gives the lane.
    uint32_t bt_rd[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int d = lane % 32;
        const int row = wn * T::TN + 16 * j + 64 * (d / 16) + d % 16;
#pragma unroll
        for (int h = 0; h < 2; ++h) bt_rd[j][h] = row * 64 + (((2 * h + lane / 32) ^ a_swz(row)) * 16);
    }

    // fragments of one 16-deep half-step
    struct Frag {
        f16x8 a[T::FM];
        f16x8 b[T::FN];
    };
    // Read slot s of half-step `half` of stage S: slot 0 is A block 0, slots
    // 1..FN are the B blocks (two transposing reads each), the rest the other
    // A blocks -- the first matrix operation needs only slots 0 and 1.
    auto read_slot = [&]<int S>(int half, int s, Frag& f) {
        const char* sa = nullptr;
        if constexpr (!AP) sa = reinterpret_cast<const char*>(stage_a.template operator()<S>());
        const char* sb = reinterpret_cast<const char*>(stage_b.template operator()<S>());
        auto tr_read = [](const char* base, int row_bytes) -> f16x8 {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS i16x4*)(base));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS i16x4*)(base + 4 * row_bytes));
            return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        if (s == 0 || s > T::FN) {
            const int i = (s == 0) ? 0 : s - T::FN;
            if constexpr (AP) {
                constexpr int PS = S / 2, SP = S % 2;
                const char* pa = reinterpret_cast<const char*>(pair_a.template operator()<PS>());
                f.a[i] = *reinterpret_cast<const f16x8*>(pa + (ap_rd[half] ^ (64u * SP)) + i * 32 * 128);
            } else if constexpr (!TA) f.a[i] = *reinterpret_cast<const f16x8*>(sa + a_rd[half] + i * 32 * 64);
            else f.a[i] = tr_read(sa + at_rd[i] + half * 16 * (T::BM * 2), T::BM * 2);
        } else {
            const int j = s - 1;
            if constexpr (!TB) f.b[j] = tr_read(sb + b_rd[j % 4] + (j / 4) * 256 + half * 16 * T::B_ROW_BYTES,
                                                T::B_ROW_BYTES);
            else f.b[j] = *reinterpret_cast<const f16x8*>(sb + bt_rd[j % 4][half] + (j / 4) * 128 * 64);
        }
    };

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Matrix op u of a half-step takes A block i = u / FN and B block j in
    // serpentine order (j runs backwards on odd i), so that from one op to
    // the next only one operand changes: at this power limit, operand bits
    // that toggle between ops cost clock (the same results, 0.7 % less time
    // under sustained load).
    auto mma_one = [&](const Frag& f, int u) {
        const int i = u / T::FN, jj = u % T::FN, j = (i & 1) ? T::FN - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
    };

    // Wait until this wave's loads older than the newest `N` are in LDS and its
    // LDS reads are done, then meet the other waves.
    auto sync = [&]<int N>() {
        static_assert(N >= 0 && N < 64, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // The ring runs for nkr = nk rounded up to a multiple of STAGES steps, so
    // that the STAGES-way unrolled loop has no exits and no branch around the
    // matrix operations (such branches make the register allocator copy the
    // whole accumulator). The extra steps multiply zero tiles.
    constexpr int R = T::STAGES, AHEAD = T::STAGES - 1;  // loads run AHEAD steps ahead
    const int nkr = (nk + R - 1) / R * R;
    Frag x, y;
    Cursor cur = cursor_at(0);  // the next step to load
    Rsrc r, rn;                 // its descriptors, and the following step's

    // The code of region kt (S = kt % R): 2 * NMMA matrix ops, those of step
    // kt, second half (fragments y), then those of step kt+1, first half
    // (fragments x). Position q of the region is one matrix op followed by
    // the memory items RegionPlan puts there:
    //  * before position kPre: the barrier. This wave's loads of step kt+1
    //    have landed (later steps may still be in flight) and its fragment
    //    reads are done, and after it every wave's have. The first kPre ops of y do not depend on it and are
    //    issued first, so the matrix cores have work while the waves meet.
    //  * then the read slots of step kt+1's first half (into x, needed by
    //    block x), from the start of block x the read slots of its second
    //    half (into y), and the loads of step kt+AHEAD spread over the region;
    //  * from position kAdv on, one item per position: the cursor moves on
    //    and the descriptors of step kt+AHEAD+1 are made for the next region
    //    (a short run of scalar instructions per position, which issue while
    //    the matrix ops run); they replace the current ones after the last
    //    load.
    // A wave issues instructions in order, so whatever sits between two
    // matrix ops must issue within one op's 32 cycles or the matrix core
    // idles; the four waves' 32 one-kilobyte direct-to-LDS loads of a step,
    // issued in a burst, held the matrix ops behind them for ~260 cycles.
    // The loads of step kt+AHEAD overwrite the stage of step kt-1, which
    // every wave finished reading before this barrier.
    constexpr int kPre = (T::NMMA - 1 - T::NSLOT) < 2 ? (T::NMMA - 1 - T::NSLOT) : 2;
    using Plan = RegionPlan<T::NMMA, T::NSLOT, T::LPT, kPre>;
    static_assert(kPre >= 0 && Plan::fits(), "the region has too few matrix ops for its reads and loads");
    constexpr Plan plan;
    constexpr int kNext = 2 * T::NMMA - 1;
    constexpr int kAdv = kPre + 1 + T::NSLOT;
    static_assert(kAdv + 3 < kNext, "the region has room for the cursor");
    // Paired A: even regions load B of steps kt+3 and kt+4, odd regions the
    // A pair of steps kt+3 and kt+4, so that both carry about as many loads.
    // Step kt+4's B uses the descriptors the cursor makes in this region:
    // those loads come after them (positions kLate on, several to a
    // position where the region is short), into the stage of step kt, which
    // no wave reads in region kt.
    constexpr int kLate = kAdv + 4;
    using PlanE = LoadSpread<T::NMMA, kPre + 1, kLate, T::B_LOADS_W>;
    using PlanL = LoadSpread<T::NMMA, kLate, 2 * T::NMMA, T::B_LOADS_W>;
    using PlanO = RegionPlan<T::NMMA, T::NSLOT, T::AP_LOADS_W, kPre>;
    static_assert(!AP || PlanO::fits(), "the region has too few matrix ops for its reads and loads");
    constexpr PlanE plan_e;
    constexpr PlanL plan_l;
    constexpr PlanO plan_o;
    // Loads allowed in flight at the barrier of region kt (S = kt % R): those
    // issued after the last one step kt+1 needs. Plain: the previous region's.
    // Paired A, kt even: step kt+1's B came first in region kt-2 and its A
    // pair from region kt-3; in flight may stay region kt-2's second B (step
    // kt+2) and region kt-1's pair: B_LOADS_W + AP_LOADS_W. kt odd: step
    // kt+1's B came second in region kt-3 and its pair from region kt-2; in
    // flight may stay region kt-1's two B steps: 2 B_LOADS_W.
    auto wait_count = [](int s) constexpr -> int {
        if constexpr (AP) return s % 2 == 1 ? 2 * T::B_LOADS_W : T::B_LOADS_W + T::AP_LOADS_W;
        else return (AHEAD - 2) * T::LPT;
    };
    auto region = [&]<int S>() {
        constexpr int S1 = (S + 1) % R, SL = (S + AHEAD) % R;
#pragma unroll
        for (int q = 0; q < 2 * T::NMMA; ++q) {
            // step kt+1 has landed (steps up to kt+AHEAD-1 may still be in flight)
            if (q == kPre) sync.template operator()<wait_count(S)>();
            if (q < T::NMMA) mma_one(y, q);
            else mma_one(x, q - T::NMMA);
            if constexpr (!AP) {
                if (plan.load[q] >= 0) load_one.template operator()<SL>(plan.load[q], r);
            } else if constexpr (S % 2 == 0) {
                for (int j = plan_e.first[q]; j < plan_e.first[q] + plan_e.count[q]; ++j)
                    load_b.template operator()<SL>(j, r);
                for (int j = plan_l.first[q]; j < plan_l.first[q] + plan_l.count[q]; ++j)
                    load_b.template operator()<S>(j, rn);
            } else {
                if (plan_o.load[q] >= 0) load_pair.template operator()<SL / 2>(plan_o.load[q], r);
            }
            if (plan.readx[q] >= 0) read_slot.template operator()<S1>(0, plan.readx[q], x);
            if (plan.ready[q] >= 0) read_slot.template operator()<S1>(1, plan.ready[q], y);
            if (q == kAdv) advance(cur);
            if (q == kAdv + 1) rn.a = desc_a(cur);
            if (q == kAdv + 3) {
                rn.b = desc_b(cur);
                rn.kleft = cur.kt < nk ? K - cur.s * T::BK : 0;
            }
            if (q == kNext) r = rn;
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (nkr > 0) {
        // prologue: steps 0..AHEAD-1 in flight; wait for step 0, read both
        // of its halves and run its first half
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (
                [&] {
                    const Rsrc r0 = descriptors(cur);
                    if constexpr (!AP) {
#pragma unroll
                        for (int i = 0; i < T::LPT; ++i) load_one.template operator()<I>(i, r0);
                    } else {
                        // steps 0 and 2 bring their A pairs, then every step its B
                        if constexpr (I % 2 == 0) {
#pragma unroll
                            for (int v = 0; v < T::AP_LOADS_W; ++v) load_pair.template operator()<I / 2>(v, r0);
                        }
#pragma unroll
                        for (int j = 0; j < T::B_LOADS_W; ++j) load_b.template operator()<I>(j, r0);
                    }
                    advance(cur);
                }(),
                ...);
        }(std::make_integer_sequence<int, AHEAD>{});
        r = descriptors(cur);
        // step 0 has landed: in flight may stay what came after its B (plain:
        // steps 1 and 2; paired: B(1), the pair of steps 2-3 and B(2))
        sync.template operator()<AP ? 2 * T::B_LOADS_W + T::AP_LOADS_W : (AHEAD - 1) * T::LPT>();
        GR_STAMP(1);
#pragma unroll
        for (int s = 0; s < T::NSLOT; ++s) read_slot.template operator()<0>(0, s, x);
#pragma unroll
        for (int u = 0; u < T::NMMA; ++u) {
            mma_one(x, u);
            if (u < T::NSLOT) read_slot.template operator()<0>(1, u, y);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Each pass of this loop runs R regions; the last region of the last
    // pass multiplies the first half of step nkr, a zero tile.
    for (int kt = 0; kt < nkr; kt += R) {
        [&]<int... S>(std::integer_sequence<int, S...>) {
            (region.template operator()<S>(), ...);
        }(std::make_integer_sequence<int, R>{});
    }
    // the zero-filling loads past the end must land, and every wave must be
    // done with its fragment reads, before the ring is reused
    sync.template operator()<0>();
    GR_STAMP(2);

    // ---- epilogue: ReLU (or bias + GELU), fp16 (nearest even) into LDS, then
    // row stores ----
    // Lane holds, for result rows d = 8q + 4*(lane/32) + r (r = 0..3), the
    // column 16*(j%4) + 64*(q/2) + 8*(q%2) + 4*(lane/32) + r of unit j/4.
    // C rows per block of the staging area: a ring slot's worth, or with
    // paired A 32 rows (16 KiB): blocks 0-3 in the B arrays, 4-5 in the
    // first pair array and 6-7 in the second (those two only for 256 rows)
    constexpr int CRS = AP ? 32 : T::C_ROWS_PER_STAGE;
    static_assert(!AP || T::B_HALVES * 2 == CRS * T::BN * 2, "a B array holds 32 rows of C");
    static_assert(!AP || T::BM <= 128 || T::BM * 64 * 2 == 2 * CRS * T::BN * 2, "a pair array holds 64 rows of C");
    auto c_stage = [&](int s) -> char* {
        if constexpr (AP) {
            char* r = reinterpret_cast<char*>(pa1) + CRS * T::BN * 2;
            r = s == 6 ? reinterpret_cast<char*>(pa1) : r;
            r = s == 5 ? reinterpret_cast<char*>(pa0) + CRS * T::BN * 2 : r;
            r = s == 4 ? reinterpret_cast<char*>(pa0) : r;
            r = s == 3 ? reinterpret_cast<char*>(sb3) : r;
            r = s == 2 ? reinterpret_cast<char*>(sb2) : r;
            r = s == 1 ? reinterpret_cast<char*>(sb1) : r;
            r = s == 0 ? reinterpret_cast<char*>(sb0) : r;
            return r;
        } else {
            char* r = reinterpret_cast<char*>(st0);
            [&]<int... I>(std::integer_sequence<int, I...>) {
                ((s == I ? (void)(r = reinterpret_cast<char*>(stage_a.template operator()<I>())) : (void)0), ...);
            }(std::make_integer_sequence<int, T::STAGES>{});
            return r;
        }
    };
    // Stores of C: 16 bytes per lane, kLanesPerRow lanes per row of the tile.
    constexpr int kRowsPerPass = T::C_ROWS_PER_PASS;  // BN / 8 lanes x 16 B per row
    constexpr int kLanesPerRow = T::BN / 8;
    constexpr int kPasses = T::BM / kRowsPerPass;
    // recomputed here from an opaque copy of the lane index: a value shared
    // with the prologue would stay live through the loop (a spilled VGPR in
    // the 256-row tiles)
    int tid_c = threadIdx.x;
    asm volatile("" : "+v"(tid_c));
    const int c = tid_c % kLanesPerRow;
    // pass `it`: this lane's row of the tile and its 16 bytes from the LDS copy
    auto pass_row = [&](int it) -> int { return it * kRowsPerPass + (int)threadIdx.x / kLanesPerRow; };
    auto pass_read = [&](int it) -> u32x4 {
        const int rl = pass_row(it);
        const char* cs = c_stage((it * kRowsPerPass) / CRS);
        return *reinterpret_cast<const u32x4*>(cs + (rl % CRS) * (T::BN * 2) + ((c ^ c_swz(rl)) * 16));
    };
    with_epilogue(p, [&]<int ACT>() {
        // the bias of this lane's columns, loaded once for all its rows
        f32x4 bias[T::FN][4];
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cl = wn * T::TN + 128 * (j / 4) + 16 * (j % 4) + 64 * (q / 2) + 8 * (q % 2) +
                               4 * (lane / 32);
                bias[j][q] = (ACT == kActBiasGelu) ? bias4(p, n0 + cl) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int rl = wm * T::TM + 32 * i + lane % 32;  // row in the tile
            // the 32 rows of block i lie in one stage array
            char* cs = c_stage(__builtin_amdgcn_readfirstlane((wm * T::TM + 32 * i) / CRS));
            char* crow = cs + (rl % CRS) * (T::BN * 2);
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = wn * T::TN + 128 * (j / 4) + 16 * (j % 4) + 64 * (q / 2) + 8 * (q % 2) +
                                   4 * (lane / 32);
                    u32x2 w;
                    w[0] = epi_pack2b<ACT>(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], bias[j][q][0], bias[j][q][1]);
                    w[1] = epi_pack2b<ACT>(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3], bias[j][q][2], bias[j][q][3]);
                    *reinterpret_cast<u32x2*>(crow + (((cl / 8) ^ c_swz(rl)) * 16) + (cl % 8) * 2) = w;
                }
            }
        }
    });
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (m0 + T::BM <= M && n0 + T::BN <= N) {
        // the whole tile is in range: each batch's LDS reads are all issued
        // before its stores, with no test per pass (a test per pass keeps each
        // store waiting for its own read)
        constexpr int kBatch = kPasses < 16 ? kPasses : 16;
        static_assert(kPasses % kBatch == 0, "store batches");
#pragma unroll
        for (int it0 = 0; it0 < kPasses; it0 += kBatch) {
            u32x4 v[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) v[b] = pass_read(it0 + b);
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                *reinterpret_cast<u32x4*>(p.C + (int64_t)(m0 + pass_row(it0 + b)) * N + n0 + c * 8) = v[b];
        }
    } else {
#pragma unroll
        for (int it = 0; it < kPasses; ++it) {
            const u32x4 v = pass_read(it);
            const int m = m0 + pass_row(it), n = n0 + c * 8;
            if (m < M && n < N) *reinterpret_cast<u32x4*>(p.C + (int64_t)m * N + n) = v;
        }
    }
    GR_STAMP_FLUSH(p);
}

}  // namespace pipelined
}  // namespace gemm_relu

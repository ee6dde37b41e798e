// Split-K kernel for few rows (M <= 16 * MB): the skinny, decode-like case.
//
// Same computation as the TileLang GEMM + ReLU example ("Writing
// high-performance kernels in TileLang", section "Escribamos un GEMM"):
// C = fp16(max(A @ B, 0)) with fp32 accumulation. With M this small the
// whole cost is streaming B from HBM once; the matrix cores are nearly idle.
// The design keeps as many bytes of B in flight as the chip allows and
// touches nothing twice:
//
//  * A workgroup owns 16 * MB rows and TN = 128 columns of C (two halves of
//    64 from neighbouring tiles' strips when B is K x N and N % 256 == 0)
//    and one range of K; each of its
//    four waves takes a quarter of that range (the reduction is split three
//    ways: inside an MFMA, across the waves, across workgroups). Splitting K
//    across CUs when the other dimensions are too small to fill the chip is
//    the split-and-combine idea of the pages' decode kernel ("Ahora uno
//    real: MLA decode"), applied here to the GEMM's reduction.
//  * B goes straight to registers: each lane loads eight consecutive rows of
//    eight consecutive columns (8 x 16 bytes; a load instruction covers four
//    rows x 256 contiguous bytes) and transposes the 8 x 8 block in registers,
//    which yields k-contiguous operands for v_mfma_f32_16x16x32_f16 without a
//    trip through LDS. D steps of 32 rows are in flight per wave (the
//    library uses 2).
//  * The B fragment is the first MFMA operand. Matrix op e of a lane uses the
//    columns 8 * (lane % 16) + e, so the sixteen results of one op are spread
//    with stride 8, and after the eight ops each lane holds 32 consecutive
//    columns of one row of C.
//  * Rows of B past the wave's range, columns past N and rows of A past M
//    read as zeros (buffer descriptors and out-of-range offsets); the K tail
//    of A is masked per lane.
//  * Transposed operands: B given as N x K is already k-contiguous, so each
//    lane loads its eight columns' 8 k-values as eight 16-byte loads and
//    skips the register transpose; A given as K x M is read one 2-byte
//    element per k (A is the small operand here).
//  * Reduction: the four waves add their fp32 tiles through LDS in a fixed
//    order. With one workgroup along K the sum goes straight to the ReLU and
//    the fp16 store. Otherwise each workgroup writes its fp32 partial tile,
//    and the last one to finish a column tile (a device-scope counter) adds
//    the partials in split order, applies the ReLU, stores fp16 C and resets
//    the counter for the next launch. The result does not depend on which
//    workgroup finishes last.
//
// Larger M is covered by more row tiles of 16 * MB rows (each re-reads B).
//
// Requirements (checked on the host): N % 8 == 0, K % 8 == 0, 16-byte
// aligned pointers, kc (the K range of a workgroup) a multiple of 4 * 32,
// M * K * 2, 8 * N * 2 and 128 * K * 2 below 2^31.
#pragma once

#include "common.hpp"

namespace gemm_relu {
namespace splitk {

// cache-policy operand of the buffer load builtin: the sc1 scope bit (device
// scope), as in the compiler's relaxed device-scope atomic accesses
constexpr int kCachePolicySc1 = 16;

template <int MB_, int NW_ = 4, int D_ = 2>
struct Cfg {
    static constexpr int MB = MB_;          // 16-row blocks
    static constexpr int BM = 16 * MB;
    static constexpr int TN = 128;          // columns of a workgroup (all its waves)
    static constexpr int NW = NW_, NT = kWave * NW;
    static constexpr int BK = 32;           // rows of B per step
    static constexpr int D = D_;            // steps in flight per wave
    static constexpr int RED_ROW = TN + 4;  // fp32 per row of the reduction buffer (padded)
    static constexpr int ROWS_PER_PASS = NT / 16;  // combine: 16 threads x 8 columns per row
    static_assert(BM % ROWS_PER_PASS == 0 || ROWS_PER_PASS % BM == 0, "combine rows");
};

template <class T, bool TA = false, bool TB = false>
__global__ void __launch_bounds__(T::NT, 1) splitk_kernel(Args p)
{
    __shared__ __attribute__((aligned(16))) float red[T::NW][T::BM][T::RED_ROW];
    __shared__ uint32_t last_flag;
    GR_STAMP_DECL;
    GR_STAMP(0);

    const int M = p.M, N = p.N, K = p.K;
    // workgroup -> (row tile, column tile, split); the splits of one tile are
    // tiles_m * tiles_n workgroups apart
    const int ntiles = p.tiles_m * p.tiles_n;
    const int tile = blockIdx.x % ntiles, ks = blockIdx.x / ntiles;
    const int tm = tile / p.tiles_n, tn = tile % p.tiles_n;
    const int m0 = tm * T::BM, n0 = tn * T::TN;
    // Logical column lc (0..127) of the tile -> column of C. With B stored
    // K x N and whole pairs of tiles (N % 256 == 0), the first 64 columns
    // come from this tile's 256-byte strip of each row of B and the last 64
    // from the neighbouring tile's: a workgroup's rate depends on where its
    // strip sits in a row (the memory channels behind it), and mixing two
    // strips evens the workgroups out. Otherwise the columns are n0 + lc.
    const bool halves = !TB && N % (2 * T::TN) == 0;
    auto gcol = [&](int lc) -> int { return (halves && lc >= T::TN / 2) ? (tn ^ 1) * T::TN + lc : n0 + lc; };
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kw = p.kc / T::NW;
    const int kbeg = min(K, ks * p.kc + wave * kw);
    const int kend = min(K, kbeg + kw);
    const int nsteps = (kend - kbeg + T::BK - 1) / T::BK;

    const int g = lane / 16, i16 = lane % 16;
    // B: lane reads rows 8g + r (r = 0..7) of a step, columns ncol .. ncol+7
    const int ncol = gcol(8 * i16);
    // (B given as N x K: rows k .. k+7 of column ncol + r, relative to
    // B + n0*K + k0)
    uint32_t boff[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if constexpr (!TB) boff[r] = (ncol < N) ? (uint32_t)((8 * g + r) * N + ncol) * 2u : kOOB;
        else boff[r] = (ncol + r < N) ? (uint32_t)((8 * i16 + r) * K + 8 * g) * 2u : kOOB;
    }
    // A: lane reads row m0 + mb*16 + i16, k-chunk 8g of a step
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint64_t)M * K * 2);
    uint32_t arow[T::MB];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        const int m = m0 + mb * 16 + i16;
        // A given as K x M: the element offset of column m (k added per step)
        arow[mb] = (m < M) ? (TA ? (uint32_t)m * 2u : (uint32_t)m * (uint32_t)K * 2u) : kOOB;
    }

    u32x4 bst[T::D][8];
    u32x4 ast[T::D][T::MB];
    // Loads of step s (rows kbeg + 32 s ...) into register slot d. Steps at
    // or past the end of the range get an empty descriptor (zeros).
    // Row tiles that share this column tile's B start their walk over the
    // wave's K range at different steps (tm mod steps, wrapping around), so
    // they do not all request the same lines of B at once: 1000 x 1016 x 1000
    // 12.1 -> 11.5 us. (With one row tile, as for few rows, nothing moves.)
    const int kskew = nsteps > 0 ? tm % nsteps : 0;
    auto issue = [&](int d, int s) {
        const int k0 = kbeg + (s < nsteps ? (s + kskew) % nsteps : s) * T::BK;
        const int64_t rows = (int64_t)kend - k0;
        if constexpr (!TB) {
            const int64_t brem = (rows > 0 ? rows : 0) * N * 2;
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (int64_t)min(k0, K) * N, (uint64_t)brem);
#pragma unroll
            for (int r = 0; r < 8; ++r) bst[d][r] = load16(rb, boff[r]);
        } else {
            // columns of this tile, k from k0: a row's 16 bytes lie past the
            // range's end only when the whole step does (kend - k0 is a
            // multiple of 8), so a step past the end loads zeros
            const int kk = min(k0, K);
            const int64_t brem = rows > 0 ? ((int64_t)(N - n0) * K - kk) * 2 : 0;
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (int64_t)n0 * K + kk, (uint64_t)brem);
            const bool live = 8 * g < rows;
#pragma unroll
            for (int r = 0; r < 8; ++r) bst[d][r] = load16(rb, live ? boff[r] : kOOB);
        }
        const int ka = k0 + 8 * g;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            if constexpr (!TA) {
                const uint32_t off = (ka < kend && arow[mb] != kOOB) ? arow[mb] + (uint32_t)ka * 2u : kOOB;
                ast[d][mb] = load16(ra, off);
            } else {
                uint16_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = ka + e < kend && arow[mb] != kOOB;
                    h[e] = ok ? p.A[(int64_t)(ka + e) * M + (arow[mb] >> 1)] : (uint16_t)0;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) ast[d][mb][j] = (uint32_t)h[2 * j] | ((uint32_t)h[2 * j + 1] << 16);
            }
        }
    };

    f32x4 acc[T::MB][8];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[mb][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int d) {
        u32x4 cols[8];
        if constexpr (!TB) transpose8x8(bst[d], cols);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) cols[e] = bst[d][e];
        }
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            const f16x8 a = __builtin_bit_cast(f16x8, ast[d][mb]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[mb][e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, cols[e]), a,
                                                                   acc[mb][e], 0, 0, 0);
        }
    };

    // Register ring of D steps: step s lives in slot s % D. The order of the
    // loads is pinned (scheduling barriers), so that when slot d is consumed
    // its loads are the oldest outstanding ones and the wait before it leaves
    // the other D - 1 steps in flight.
#pragma unroll
    for (int d = 0; d < T::D; ++d) {
        issue(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = 0; s0 < nsteps; s0 += T::D) {
#pragma unroll
        for (int d = 0; d < T::D; ++d) {
            compute(d);
#ifdef GR_STAMPS
            if (s0 == 0 && d == 0) GR_STAMP(1);
#endif
            __builtin_amdgcn_sched_barrier(0);
            issue(d, s0 + d + T::D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    GR_STAMP(2);
    // ---- reduction across the four waves (fixed order) ----
    // Lane holds acc[mb][e][r] = C[mb*16 + i16][gcol(32g + 8r + e)].
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        float* row = &red[wave][mb * 16 + i16][32 * g];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<f32x4*>(row + 8 * r) = f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            *reinterpret_cast<f32x4*>(row + 8 * r + 4) =
                f32x4{acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
        }
    }
    __syncthreads();
    // Combine: thread t adds the waves' values for rows m0 + t/16 + j*RP
    // (j = 0, 1, ...), logical columns 8*(t%16) .. +7 of the tile.
    constexpr int RP = T::ROWS_PER_PASS;
    constexpr int NJ = (T::BM + RP - 1) / RP;
    const int t = threadIdx.x;
    const int cm = t / 16, cn = 8 * (t % 16);
    const int n = gcol(cn);
    float v[NJ][8];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
        const int rl = cm + j * RP;  // row in the tile
        if (rl < T::BM) {
#pragma unroll
            for (int w = 0; w < T::NW; ++w) {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(&red[w][rl][cn]);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(&red[w][rl][cn + 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[j][e] += lo[e];
                    v[j][e + 4] += hi[e];
                }
            }
        }
    }

    // ReLU (or bias + GELU), fp16 (nearest even), 16-byte stores
    auto store_c = [&](const float (&vals)[NJ][8]) {
        with_epilogue(p, [&]<int ACT>() {
            // the bias of this thread's 8 columns, loaded once for all its rows
            f32x4 blo = f32x4{0.f, 0.f, 0.f, 0.f}, bhi = blo;
            if constexpr (ACT == kActBiasGelu) {
                blo = bias4(p, n);
                bhi = bias4(p, n + 4);
            }
            const float bv[8] = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int rl = cm + j * RP, m = m0 + rl;
                if (rl < T::BM && m < M && n < N) {
                    u32x4 h;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        h[q] = epi_pack2b<ACT>(vals[j][2 * q], vals[j][2 * q + 1], bv[2 * q], bv[2 * q + 1]);
                    *reinterpret_cast<u32x4*>(p.C + (int64_t)m * N + n) = h;
                }
            }
        });
    };

    if (p.splits == 1) {
        store_c(v);
        GR_STAMP_FLUSH(p);
        return;
    }

    // ---- split across workgroups: partials, then the last workgroup combines ----
    // The eight XCDs each have their own L2, and a device-wide fence would
    // write back or invalidate a whole L2 per workgroup. Instead every access
    // to the shared data (partials, counter) carries the device-scope cache
    // policy (sc1, as the compiler's device-scope atomics do), which the
    // hardware performs at the level the XCDs share: the partials are stored
    // that way, this wave waits until its stores are acknowledged
    // (vmcnt(0)), the workgroup meets, and only then one lane counts the
    // workgroup in (a device-scope atomic). The last workgroup reads the
    // partials with device-scope loads, all issued after it saw the final
    // count.
    // Why this order holds without release/acquire at device scope:
    //  * hardware: a device-scope store is acknowledged (and vmcnt drops) only
    //    once it is visible at the level the XCDs share, and device-scope
    //    atomics and loads are performed at that level too. So when a
    //    workgroup's count lands, all of its partials are already visible
    //    there, and the last workgroup's loads, issued after its count
    //    returned, read them from there;
    //  * compiler: the asm stores may not sink below the empty asm with
    //    a memory clobber that sits before the vmcnt(0) wait, and the wait
    //    and the volatile asm keep their order; the barrier's
    //    workgroup-scope fences keep the count after the wait, and the
    //    last workgroup's loads after the barrier that publishes the count
    //    (and they depend on it through the branch on last_flag).
    // Partials are stored 16 bytes at a time with the device-scope cache
    // policy (sc1): the instruction the compiler emits for a relaxed
    // device-scope atomic store, which it does not offer wider than 8 bytes.
    // Each dword is stored with device scope; nothing reads a partial before
    // the count below, so the 16 bytes need not land as one. A store of more
    // than 8 bytes reads its data registers after issue: an instruction that
    // writes them must wait one cycle, which the compiler ensures for its own
    // stores but not around inline asm, hence the s_nop in each.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int rl = cm + j * RP, m = m0 + rl;
        if (rl < T::BM && m < M && n < N) {
            float* dst = p.partial + ((int64_t)ks * M + m) * N + n;
            const u32x4 lo = __builtin_bit_cast(u32x4, f32x4{v[j][0], v[j][1], v[j][2], v[j][3]});
            const u32x4 hi = __builtin_bit_cast(u32x4, f32x4{v[j][4], v[j][5], v[j][6], v[j][7]});
            asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(lo) : "memory");
            asm volatile("global_store_dwordx4 %0, %1, off offset:16 sc1\n\ts_nop 1" ::"v"(dst), "v"(hi) : "memory");
        }
    }
    asm volatile("" ::: "memory");  // the stores above stay above the wait
    wait_vmcnt<0>();                 // this wave's partial stores are acknowledged
    asm volatile("" ::: "memory");
    __syncthreads();
    if (t == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == (uint32_t)(p.splits - 1)) ? 1u : 0u;
    }
    __syncthreads();
    GR_STAMP(4);
    if (!last_flag) {
        GR_STAMP_FLUSH(p);
        return;
    }
    constexpr int kBatch = 8;
    float sum[NJ][8];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[j][e] = 0.f;
    // The partials are read 16 bytes at a time with the device-scope cache
    // policy (sc1, what a relaxed device-scope atomic load compiles to),
    // through one buffer descriptor per split: the host splits K only when
    // one split's M x N fp32 partials stay below 2^31 bytes. Up to kBatch
    // splits are loaded before any is added (their latencies overlap); the
    // additions keep split order.
    for (int q0 = 0; q0 < p.splits; q0 += kBatch) {
        u32x4 buf[kBatch][NJ][2];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int q = q0 + b;
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(p.partial + (int64_t)(q < p.splits ? q : 0) * M * N, (uint64_t)M * N * 4);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int rl = cm + j * RP, m = m0 + rl;
                const bool ok = q < p.splits && rl < T::BM && m < M && n < N;
                const uint32_t off = ok ? ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 4u : kOOB;
                buf[b][j][0] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, 0, kCachePolicySc1);
                buf[b][j][1] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + 16u), 0, kCachePolicySc1);
            }
        }
        // (each element is copied out before the cast: this compiler's
        // __builtin_bit_cast of a vector element reads element 0 whatever
        // the index)
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = buf[b][j][e / 4][e % 4];
                    sum[j][e] += __builtin_bit_cast(float, w);
                }
    }
    store_c(sum);
    if (t == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    GR_STAMP_FLUSH(p);
}

}  // namespace splitk
}  // namespace gemm_relu

// Row softmax and the attention forward pass on gfx950: the second workload
// of "TileLang simplifica la creación de kernels GPU de alto rendimiento"
// (section "Softmax y FlashAttention sin materializar matrices
// innecesarias"), on the same MFMA core and load machinery as the GEMM.
#pragma once

#include "common.hpp"

namespace gemm_relu {
namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float h2f(uint32_t w, int hi)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? (w >> 16) : (w & 0xFFFF)));
}

__device__ __forceinline__ uint32_t f2h2(float lo, float hi)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// ---------------------------------------------------------------------------
// Row softmax: y = exp(x - max) / sum exp(x - max), per row, in fp32, fp16 out
// (round to nearest even).
// ---------------------------------------------------------------------------

struct SoftmaxArgs {
    const uint16_t* X;
    uint16_t* Y;
    int rows, cols;
};

// One wave per row, the row held in registers: each lane takes V chunks of 8
// columns (chunk c = lane + 64 v, so a wave's loads and stores are contiguous
// 1 KiB runs). The row is read once and written once: HBM-bound.
// Requirements: cols % 8 == 0, cols <= 512 V, 16-byte aligned X and Y.
template <int V>
__global__ void __launch_bounds__(256) softmax_rows_vec(SoftmaxArgs a)
{
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int row = blockIdx.x * 4 + wave;
    if (row >= a.rows) return;  // the whole wave leaves together
    const int cols = a.cols;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X + (int64_t)row * cols, (uint64_t)cols * 2);
    u32x4 raw[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int c = lane + kWave * v;
        raw[v] = load16(rx, c * 8 < cols ? (uint32_t)c * 16u : kOOB);
    }
    float f[V][8];
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const bool live = (lane + kWave * v) * 8 < cols;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f[v][e] = live ? h2f(raw[v][e / 2], e % 2) : -INFINITY;
            m = fmaxf(m, f[v][e]);
        }
    }
    m = wave_max(m);
    const float mb = m * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f[v][e] = exp2_fast(fmaf(f[v][e], kLog2e, -mb));
            s += f[v][e];
        }
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int c = lane + kWave * v;
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = f2h2(f[v][2 * j] * inv, f[v][2 * j + 1] * inv);
        if (c * 8 < cols) *reinterpret_cast<u32x4*>(a.Y + (int64_t)row * cols + c * 8) = w;
    }
}

// Any shape and alignment: one workgroup per row, element-wise. Pass 1 keeps a
// running (maximum, sum) per thread -- the sum rescaled whenever the maximum
// grows -- and combines the threads' pairs; pass 2 reads the row again and
// writes it.
__global__ void __launch_bounds__(256) softmax_rows_any(SoftmaxArgs a)
{
    __shared__ float red_m[256], red_s[256];
    const int row = blockIdx.x, t = threadIdx.x;
    const int cols = a.cols;
    const uint16_t* x = a.X + (int64_t)row * cols;
    float m = -INFINITY, s = 0.f;
    for (int j = t; j < cols; j += 256) {
        const float v = (float)__builtin_bit_cast(_Float16, x[j]) * kLog2e;
        if (v > m) {
            s = s * exp2_fast(m - v) + 1.0f;
            m = v;
        } else {
            s += exp2_fast(v - m);
        }
    }
    red_m[t] = m;
    red_s[t] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (t < w) {
            const float m1 = red_m[t], m2 = red_m[t + w];
            const float mm = fmaxf(m1, m2);
            const float s1 = m1 == -INFINITY ? 0.f : red_s[t] * exp2_fast(m1 - mm);
            const float s2 = m2 == -INFINITY ? 0.f : red_s[t + w] * exp2_fast(m2 - mm);
            red_m[t] = mm;
            red_s[t] = s1 + s2;
        }
        __syncthreads();
    }
    const float M = red_m[0], inv = 1.0f / red_s[0];
    uint16_t* y = a.Y + (int64_t)row * cols;
    for (int j = t; j < cols; j += 256) {
        const float v = (float)__builtin_bit_cast(_Float16, x[j]) * kLog2e;
        y[j] = __builtin_bit_cast(uint16_t, (_Float16)(exp2_fast(v - M) * inv));
    }
}

// ---------------------------------------------------------------------------
// Attention forward (the FlashAttention scheme: query tiles stream over key /
// value tiles with a running maximum and sum, and the score matrix never goes
// to memory).
//
//  * A workgroup owns BM = 32 NW query rows of one (batch, head): NW waves of
//    32 rows, two waves per SIMD. With NW = 4 two workgroups share a CU and
//    run out of step with each other, so one's softmax arithmetic overlaps
//    the other's matrix ops, and the small workgroup evens out causal work;
//    with NW = 8 (D = 128 without the mask) one workgroup fills the CU and
//    each K and V tile is loaded into LDS once for 256 query rows.
//  * Key and value tiles of BN = 64 rows go global -> LDS with direct 1 KiB
//    buffer loads into two LDS stages (one array per stage and operand), the
//    next tile in flight while the current one is used; rows past the
//    sequence read as zeros.
//  * S = Q K^T on v_mfma_f32_32x32x16_f16 with the K fragment first: each lane
//    ends up with one query row (lane % 32) and 16 of the tile's keys. Q's
//    fragments stay in registers for the whole pass.
//  * Online softmax per row in the log2 domain: t = s * scale * log2(e),
//    p = 2^(t - m), l += sum p, O += P V, with the reference m of each row
//    moved to the running maximum (and O, l rescaled by 2^(m - m')) only when
//    a score exceeds it by more than 2^8 -- exact in real arithmetic, and it
//    spares most tiles the rescaling. The row's two lanes (lane, lane ^ 32)
//    meet with one swap for the maximum; the sums stay per lane until the
//    end. Interior tiles fold the scaling into the exponent (one FMA per
//    score); only tiles at the sequence end or the causal diagonal mask.
//  * O += P V with P as the second operand straight from the S registers
//    (converted to fp16): the lane already holds, for each 16-deep chunk of
//    keys, the 8 values the operand wants -- in the key order {0-3, 8-11} or
//    {4-7, 12-15} -- so the value tile is read with the transposing LDS load
//    in that same key order, and no data moves between lanes.
//  * Causal: query i sees keys j <= i. A workgroup stops at the last tile its
//    rows can see; tiles that cross the diagonal (or the sequence end) are
//    masked to -inf before the maximum.
//  * End: O / l to fp16 (nearest even); optionally the log-sum-exp m + ln l.
//
// Layout: Q, O [BH][Sq][D], K, V [BH][Skv][D], contiguous fp16; lse [BH][Sq]
// fp32. Requirements: D in {64, 128}, 16-byte aligned pointers.
// ---------------------------------------------------------------------------

struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    uint16_t* O;
    float* lse;  // may be null
    int BH, Sq, Skv;
    float scale_log2;  // softmax scale * log2(e)
    int causal;
    int nqb;    // query tiles per (batch, head)
    int npair;  // work items per (batch, head): (nqb + 1) / 2 when paired, else nqb
    int paired; // 1: an item runs two query tiles (causal); 0: one
};

template <int D_, int NW_ = 8>
struct AttnCfg {
    static constexpr int D = D_;
    static constexpr int NW = NW_, BM = 32 * NW, BN = 64, NT = NW * kWave;
    static constexpr int KK = D / 16;             // 16-deep chunks of the QK^T reduction
    static constexpr int DB = D / 32;             // 32-wide blocks of O columns
    static constexpr int CPR = D / 8;             // 16-byte chunks per K / V row
    static constexpr int RPL = kWave / CPR;       // rows per 1 KiB load
    static constexpr int LOADS = BN * D * 2 / 1024;  // 1 KiB loads per tile
    static constexpr int LW = LOADS / NW;            // per wave, per tile
    static constexpr int TILE_HALVES = BN * D;
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    static_assert(LOADS % NW == 0, "loads split evenly over the waves");
};

// K tile: row r, logical chunk c at physical chunk c ^ k_swz(r). The
// fragment reads take 16 consecutive rows at one chunk: with 256-byte rows
// (D = 128) XOR-ing with r % 16 puts them on 16 chunks; with 128-byte rows two
// rows share a 256-byte bank window, and r / 2 does the same.
template <int D>
__device__ __forceinline__ int k_swz(int r)
{
    if constexpr (D == 128) return r & 15;
    else return (r >> 1) & 7;
}

// V tile: read with transposing loads, four consecutive rows at a 32-byte
// column pair and the next pair for the other 16-lane group; moving the pair
// by 2 (r % 4) (D = 128) or 2 ((r / 2) % 2) (D = 64) spreads them over the
// banks.
template <int D>
__device__ __forceinline__ int v_swz(int r)
{
    if constexpr (D == 128) return 4 * (r & 3);
    else return 4 * ((r >> 1) & 1);
}

// One query tile (BM rows) of batch-head bh against all its keys, in the
// workgroup's four LDS stages.
template <class T>
__device__ __forceinline__ void attn_tile(const AttnArgs& p, int bh, int qb, uint16_t* ks0, uint16_t* ks1,
                                          uint16_t* vs0, uint16_t* vs1)
{
    constexpr int D = T::D;
    const int Sq = p.Sq, Skv = p.Skv;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int q0 = qb * T::BM;            // first query row of the workgroup
    const int qw = q0 + wave * 32;        // first row of this wave
    const int qrow = qw + lane % 32;      // this lane's row
    const int hi = lane / 32;

    // key tiles this workgroup needs
    int nkb = (Skv + T::BN - 1) / T::BN;
    if (p.causal) {
        const int last = min(Sq, q0 + T::BM) - 1;  // last query row of the workgroup
        nkb = min(nkb, last / T::BN + 1);
    }
    const int nkb2 = (nkb + 1) / 2 * 2;  // the loop runs pairs of tiles; a padding tile is fully masked

    const uint16_t* Kh = p.K + (int64_t)bh * Skv * D;
    const uint16_t* Vh = p.V + (int64_t)bh * Skv * D;

    // ---- Q fragments, kept in registers: row qrow, columns 16 kk + 8 hi .. +7.
    // A negative scale is moved onto Q: the sign bits are flipped, which
    // negates every score exactly, and the exponents use |scale|. So the
    // row reference is always a maximum.
    const float c = fabsf(p.scale_log2);
    f16x8 qf[T::KK];
    {
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(p.Q + (int64_t)bh * Sq * D, (uint64_t)Sq * D * 2);
        const uint32_t flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
            const uint32_t off = qrow < Sq ? (uint32_t)(qrow * D + 16 * kk + 8 * hi) * 2u : kOOB;
            qf[kk] = __builtin_bit_cast(f16x8, load16(rq, off) ^ flip);
        }
    }

    // ---- direct loads of key / value tile j into stage S
    // load i of a tile: rows i*RPL + lane / CPR, physical chunk lane % CPR.
    // The descriptor of tile j ends at the last key: a row past it lies
    // wholly beyond the descriptor's range and reads as zeros.
    uint32_t koff[T::LW], voff[T::LW];
#pragma unroll
    for (int i = 0; i < T::LW; ++i) {
        const int gi = wave * T::LW + i;
        const int r = gi * T::RPL + lane / T::CPR;
        const int pc = lane % T::CPR;
        koff[i] = (uint32_t)(r * D + 8 * (pc ^ k_swz<D>(r))) * 2u;
        voff[i] = (uint32_t)(r * D + 8 * (pc ^ v_swz<D>(r))) * 2u;
    }
    // K tile j into K stage S, V tile j into V stage S
    auto issue_k = [&]<int S>(int j) {
        const int kv0 = j * T::BN;
        const bool live = j < nkb;
        const uint64_t bytes = live ? (uint64_t)(Skv - kv0) * D * 2 : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (int64_t)(live ? kv0 : 0) * D, bytes);
        uint16_t* kd = S == 0 ? ks0 : ks1;
#pragma unroll
        for (int i = 0; i < T::LW; ++i) {
            const int gi = wave * T::LW + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (GR_LDS void*)(kd + gi * 512), 16, (int)koff[i], 0, 0, 0);
        }
    };
    auto issue_v = [&]<int S>(int j) {
        const int kv0 = j * T::BN;
        const bool live = j < nkb;
        const uint64_t bytes = live ? (uint64_t)(Skv - kv0) * D * 2 : 0;
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (int64_t)(live ? kv0 : 0) * D, bytes);
        uint16_t* vd = S == 0 ? vs0 : vs1;
#pragma unroll
        for (int i = 0; i < T::LW; ++i) {
            const int gi = wave * T::LW + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (GR_LDS void*)(vd + gi * 512), 16, (int)voff[i], 0, 0, 0);
        }
    };

    // ---- per-lane LDS byte offsets of the fragment reads
    // K fragment (jb, kk): row 32 jb + lane % 32, logical chunk 2 kk + hi
    uint32_t krd[2][T::KK];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
            const int r = 32 * jb + lane % 32;
            krd[jb][kk] = (uint32_t)(r * D * 2 + 16 * ((2 * kk + hi) ^ k_swz<D>(r)));
        }
    // V fragment (c, db), transposing read t: the 16-lane group g reads rows
    // 16 c + 4 (g / 2) + 8 t + (lane % 16) / 4 and columns 32 db + 16 (g % 2) +
    // 4 (lane % 4) .. +3; after the transpose the lane holds column
    // 32 db + lane % 32 for four keys -- the keys its P values belong to.
    const int g = lane / 16, q16 = lane % 16;
    uint32_t vrd[4][T::DB];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
            const int r = 16 * c + 4 * (g / 2) + q16 / 4;  // t = 0; t = 1 adds 8 rows, same swizzle
            const int col = 32 * db + 16 * (g % 2) + 4 * (q16 % 4);
            vrd[c][db] = (uint32_t)(r * D * 2 + 16 * ((col / 8) ^ v_swz<D>(r)) + 8 * ((col / 4) % 2));
        }

    f32x16 acc_o[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[db][e] = 0.f;
    float m_run = -INFINITY;  // running maximum of this lane's row (log2 domain)
    float l_run = 0.f;        // running sum of this lane's share of the row

    // S = Q K^T for the 64 keys of K stage S
    auto qk = [&]<int S>(f32x16 (&sc)[2]) {
        const char* kb = reinterpret_cast<const char*>(S == 0 ? ks0 : ks1);
        f16x8 kf[2][T::KK];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int kk = 0; kk < T::KK; ++kk) kf[jb][kk] = *reinterpret_cast<const f16x8*>(kb + krd[jb][kk]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[jb][e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < T::KK; ++kk)
                sc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[jb][kk], qf[kk], sc[jb], 0, 0, 0);
        }
    };

    // Both halves of the wave hold the same 32 rows (lanes l and l + 32):
    // the maximum of a value over the two.
    auto pair_max = [](float v) -> float {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    // This lane's maximum over the 32 scores of s it holds; two chains of
    // three-way maxima.
    auto lane_max = [](const f32x16 (&s)[2]) -> float {
        float a = -INFINITY, b = -INFINITY;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            a = fmaxf(a, fmaxf(s[0][2 * q], s[0][2 * q + 1]));
            b = fmaxf(b, fmaxf(s[1][2 * q], s[1][2 * q + 1]));
        }
        return fmaxf(a, b);
    };

    // The row statistics of tile j's scores s, whose lane maximum hs the
    // caller took as the scores came out of the matrix ops: keys past the
    // end, or after the row when causal, are masked (only tiles at the
    // sequence end or the diagonal need the test, and there the maximum is
    // taken again; the lane holds keys kv0 + 32 jb + 8 (e / 4) + 4 hi + e % 4),
    // and the row's reference m_run moves when needed. Returns the reference
    // the exponents use.
    auto stats = [&](int j, f32x16 (&s)[2], float hs) -> float {
        const int kv0 = j * T::BN;
        const bool edge = kv0 + T::BN > Skv || (p.causal && kv0 + T::BN - 1 > qw);
        if (edge) {
            const int lim = p.causal ? min(Skv, qrow + 1) : Skv;
            const int rel = lim - kv0 - 4 * hi;  // key offsets below rel are visible
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    s[jb][e] = (32 * jb + 8 * (e / 4) + e % 4 < rel) ? s[jb][e] : -INFINITY;
            hs = lane_max(s);
        }
        const float mt = pair_max(hs * c);
        // Lazy rescaling: p = 2^(t - m_run) with m_run, the reference of the
        // row, moved only when a scaled score t exceeds it by more than kTau
        // (then O and l are rescaled). Every p stays <= 2^kTau, so fp16 holds
        // it with the same relative precision, and O / l is unchanged in
        // exact arithmetic. A row with nothing visible yet keeps m_run = -inf.
        constexpr float kTau = 8.0f;
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kTau) != 0) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_new == m_run ? 1.0f : exp2_fast(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc_o[db][e] *= alpha;
        }
        return m_run == -INFINITY ? 0.f : m_run;
    };

    // One straight-line stretch per tile, matrix ops and VALU work
    // interleaved in a fixed order (scheduling barriers); every fragment read
    // is issued two matrix ops ahead, in a stretch of its own so that it
    // leaves before the matrix op it overlaps:
    //   phase 1: S' = Q K(next)^T from K stage SK, with the exponentials of
    //            the current tile's first 24 scores (chunks 0-2 of P) between
    //            the matrix ops;
    //   phase 2: O += P V from V stage SV, chunk by chunk, with the last 8
    //            exponentials (chunk 3) and the lane maximum of S' between
    //            the matrix ops.
    // p = 2^(s c - m): the scale folded into one FMA per score. The row sums
    // are pinned to their stretch (an empty asm statement that takes them),
    // since nothing else ties them there. Returns the lane maximum of S'.
    auto fused = [&]<int SK, int SV>(f32x16 (&s_cur)[2], f32x16 (&s_next)[2], float m_use) -> float {
        const char* kb = reinterpret_cast<const char*>(SK == 0 ? ks0 : ks1);
        const char* vb = reinterpret_cast<const char*>(SV == 0 ? vs0 : vs1);
        constexpr int NQ = 2 * T::KK;       // Q K^T matrix ops
        constexpr int NP = 4 * T::DB;       // P V matrix ops
        constexpr int EX1 = 24;             // exponentials in phase 1
        constexpr int NEX2 = 32 - EX1;      // over the first 2 DB matrix ops of phase 2
        constexpr int NMX = 16;             // three-way maxima over S'
        float ls1 = 0.f, ls2 = 0.f;
        f16x8 pf[4];
        auto expo = [&](int x, float& ls) {  // score x: block x / 16, element x % 16 -> chunk x / 8
            const float pe = exp2_fast(fmaf(s_cur[x / 16][x % 16], c, -m_use));
            ls += pe;
            pf[x / 8][x % 8] = (_Float16)pe;
        };
        // Q K^T op t: key block t % 2, reduction chunk t / 2 -- neighbouring
        // matrix ops accumulate into different registers
        auto read_k = [&](int t) -> f16x8 {
            return *reinterpret_cast<const f16x8*>(kb + krd[t % 2][t / 2]);
        };
        auto read_v = [&](int u) -> f16x8 {
            const char* base = vb + vrd[u / T::DB][u % T::DB];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS i16x4*)(base));
            const i16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GR_LDS i16x4*)(base + 8 * D * 2));
            return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7));
        };
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s_next[jb][e] = 0.f;
        f16x8 kr[NQ];
        kr[0] = read_k(0);
        kr[1] = read_k(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            if (t + 2 < NQ) kr[t + 2] = read_k(t + 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = t * EX1 / NQ; x < (t + 1) * EX1 / NQ; ++x) expo(x, ls1);
            s_next[t % 2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kr[t], qf[t / 2], s_next[t % 2], 0, 0, 0);
            asm volatile("" : "+v"(ls1));
            __builtin_amdgcn_sched_barrier(0);
        }
        f16x8 vr[NP];
        vr[0] = read_v(0);
        vr[1] = read_v(1);
        __builtin_amdgcn_sched_barrier(0);
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            if (u + 2 < NP) vr[u + 2] = read_v(u + 2);
            __builtin_amdgcn_sched_barrier(0);
            if (u < 2 * T::DB) {
#pragma unroll
                for (int x = EX1 + u * NEX2 / (2 * T::DB); x < EX1 + (u + 1) * NEX2 / (2 * T::DB); ++x) expo(x, ls2);
            }
            // S' is complete (phase 1 is over): its lane maximum, pairs of
            // scores q = 2 i, 2 i + 1 of block i / 8, alternating chains
#pragma unroll
            for (int i = u * NMX / NP; i < (u + 1) * NMX / NP; ++i) {
                float& mx = (i % 2) ? mx1 : mx0;
                const int jb = i / 8, q = i % 8;
                mx = fmaxf(mx, fmaxf(s_next[jb][2 * q], s_next[jb][2 * q + 1]));
            }
            acc_o[u % T::DB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[u], pf[u / T::DB], acc_o[u % T::DB], 0, 0, 0);
            asm volatile("" : "+v"(ls2), "+v"(mx0), "+v"(mx1));
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run += ls1 + ls2;
        return fmaxf(mx0, mx1);
    };

    // Software pipeline over key tiles, one barrier per tile. Iteration j:
    //   wait for K(j+1) and V(j) (issued one iteration earlier), barrier;
    //   issue K(j+2) and V(j+1) into the stages freed by iteration j-1;
    //   S' = Q K(j+1)^T (matrix ops), then the softmax of tile j (VALU work
    //   that runs while those matrix ops execute), then O += P V(j).
    // K and V each have two stages, offset by one tile; j runs in pairs so
    // every stage index is a compile-time constant.
    auto sync = [&]() {
        wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };
    f32x16 sa[2], sb[2];
    issue_k.template operator()<0>(0);
    issue_v.template operator()<0>(0);
    issue_k.template operator()<1>(1);
    sync();
    qk.template operator()<0>(sa);
    float hs = lane_max(sa);
    for (int j = 0; j < nkb2; j += 2) {
        sync();
        issue_k.template operator()<0>(j + 2);
        issue_v.template operator()<1>(j + 1);
        hs = fused.template operator()<1, 0>(sa, sb, stats(j, sa, hs));
        sync();
        issue_k.template operator()<1>(j + 3);
        issue_v.template operator()<0>(j + 2);
        hs = fused.template operator()<0, 1>(sb, sa, stats(j + 1, sb, hs));
    }
    wait_vmcnt<0>();  // the last (empty) loads must land before the kernel ends

    // ---- O / l, fp16 stores; lane holds row qrow, columns
    // 32 db + 8 (e / 4) + 4 hi + e % 4
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < Sq) {
        uint16_t* orow = p.O + ((int64_t)bh * Sq + qrow) * D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2 wv;
                wv[0] = f2h2(acc_o[db][4 * q4 + 0] * inv, acc_o[db][4 * q4 + 1] * inv);
                wv[1] = f2h2(acc_o[db][4 * q4 + 2] * inv, acc_o[db][4 * q4 + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * q4 + 4 * hi) = wv;
            }
        if (p.lse && hi == 0)
            p.lse[(int64_t)bh * Sq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <class T>
__global__ void __launch_bounds__(T::NT, 2) attn_fwd_kernel(AttnArgs p)  // two waves per SIMD
{
    __shared__ __attribute__((aligned(1024))) uint16_t ks0[T::TILE_HALVES];
    __shared__ __attribute__((aligned(1024))) uint16_t ks1[T::TILE_HALVES];
    __shared__ __attribute__((aligned(1024))) uint16_t vs0[T::TILE_HALVES];
    __shared__ __attribute__((aligned(1024))) uint16_t vs1[T::TILE_HALVES];

    // Work item -> (batch-head, query tiles). Items are taken in
    // XCD-contiguous ranges (die b % 8 gets one run of them), and a head's
    // items sit next to each other so they share its K and V in the die's L2.
    // Causal: item i of a head runs query tile nqb-1-i and then tile i; the
    // two together see the same number of key tiles for every i, so all
    // workgroups carry equal work (the middle tile of an odd count runs
    // alone). Without the mask every tile sees every key, and item i runs
    // tile i alone: a die's resident workgroups then cover two heads, whose
    // K and V (2 MiB each at 4096 x 128) its 4 MiB L2 holds while the
    // workgroups walk them in step, instead of four heads walked twice.
    int w = blockIdx.x;
    {
        const int nblk = gridDim.x, q = nblk / 8, r = nblk % 8;
        const int xcd = w % 8, idx = w / 8;
        w = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    }
    const int bh = w / p.npair, i = w % p.npair;
    if (!p.paired) {
        attn_tile<T>(p, bh, i, ks0, ks1, vs0, vs1);
        return;
    }
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int qb = pass == 0 ? p.nqb - 1 - i : i;
        if (pass == 1) {
            if (qb == p.nqb - 1 - i) break;
            __syncthreads();  // every wave is done with the stages before they refill
        }
        attn_tile<T>(p, bh, qb, ks0, ks1, vs0, vs1);
    }
}

}  // namespace attn
}  // namespace gemm_relu

// The sustained rate of gfx950's matrix cores on their own: every SIMD runs
// back-to-back fp16 matrix ops into fp32 accumulators, with no global memory
// traffic in the timed loop, while a host thread samples the shader clock and
// the board power from sysfs. It bounds what any fp16 GEMM can sustain on the
// same operand bits: a GEMM adds loads, LDS traffic and an epilogue to this.
//
// The GEMM + ReLU kernel's main loop ("Writing high-performance kernels in
// TileLang", section "Escribamos un GEMM") issues v_mfma_f32_32x32x16_f16 on
// 4 x 4 blocks per wave; the probe runs the same instruction and block shape
// (and, for comparison, v_mfma_f32_16x16x32_f16 on 8 x 8 blocks), with
// operands either held in registers or re-read from LDS every sweep (double
// buffered, as the GEMM reads its fragments).
//
// Operand bits: "random" draws fp16 values with a random sign, an exponent
// in [2^-2, 2^1] and a random mantissa (the magnitude range of N(0, 1)
// samples) from a SplitMix64 stream; "constant" fills every operand with 1.0.
// On random bits the chip's power limit sets the clock, on constant bits it
// does not, which is the point of running both.
//
// Usage: mfma_ceiling [seconds per case, default 1.0]
// Output: one line per case: TFLOP/s, mean shader clock (MHz), TFLOP/s per
// GHz against the 1048.6 TFLOP/s per GHz of 256 CUs x 4 SIMDs x 1024 FLOP per
// cycle (2516.6 TFLOP/s at 2.4 GHz), mean board power and energy per FLOP.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <glob.h>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;       // one wave per SIMD
constexpr int kFrags = 16;      // operand fragments per wave in LDS (8 for A, 8 for B)
constexpr int kBlocks = 256;    // one workgroup per CU
constexpr double kPerGhz = 1048.6;

#define CHECK(x)                                                                      \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));       \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

// KIND 0: 32x32x16 on 4 x 4 blocks; KIND 1: 16x16x32 on 8 x 8 blocks (256
// accumulator registers either way). LDS_FEED: operands re-read from LDS
// every sweep, the next sweep's while this one's matrix ops run.
template <int KIND, bool LDS_FEED>
__global__ void __launch_bounds__(kWaves * 64, 1) mfma_loop(const u32x4* src, int iters, float* out)
{
    __shared__ __attribute__((aligned(16))) u32x4 lds[kWaves][kFrags][64];
    constexpr int NF = KIND == 0 ? 4 : 8;  // A and B fragments per sweep
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const u32x4* mine = src + (size_t)(blockIdx.x * kWaves + wave) * kFrags * 64;
#pragma unroll
    for (int f = 0; f < kFrags; ++f) lds[wave][f][lane] = mine[f * 64 + lane];
    __syncthreads();

    f16x8 a[2][NF], b[2][NF];
    // fragment set for sweep s: A from slots (i + s) % 8, B from 8 + (i + s) % 8
    auto fetch = [&](int set, int s) {
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            a[set][i] = __builtin_bit_cast(f16x8, lds[wave][(i + s) & 7][lane]);
            b[set][i] = __builtin_bit_cast(f16x8, lds[wave][8 + ((i + s) & 7)][lane]);
        }
    };
    fetch(0, 0);
    fetch(1, 1);  // (the register-fed cases keep these two sets)

    using Acc = std::conditional_t<KIND == 0, f32x16, f32x4>;
    Acc acc[NF][NF];
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = Acc{};

    // one sweep: every block once, serpentine over B so that consecutive ops
    // share an operand
    auto sweep = [&](int set) {
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
            for (int jj = 0; jj < NF; ++jj) {
                const int j = (i & 1) ? NF - 1 - jj : jj;
                if constexpr (KIND == 0)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[set][i], b[set][j], acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[set][i], b[set][j], acc[i][j], 0, 0, 0);
            }
    };
    // each fetch is issued one sweep ahead of its use, right after the sweep
    // that last read its registers (scheduling barriers keep the order)
    for (int it = 0; it < iters; it += 2) {
        if constexpr (LDS_FEED) fetch(1, it + 1);
        __builtin_amdgcn_sched_barrier(0);
        sweep(0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LDS_FEED) fetch(0, it + 2);
        __builtin_amdgcn_sched_barrier(0);
        sweep(1);
        __builtin_amdgcn_sched_barrier(0);
    }
    // every accumulator feeds the output, so no matrix op is dead code
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int e = 0; e < (KIND == 0 ? 16 : 4); ++e) s += acc[i][j][e];
    out[blockIdx.x * kWaves * 64 + threadIdx.x] = s;
}

std::string first_match(const char* pattern)
{
    glob_t g;
    std::string r;
    if (glob(pattern, 0, nullptr, &g) == 0 && g.gl_pathc > 0) r = g.gl_pathv[0];
    globfree(&g);
    return r;
}

// current shader clock: the line of pp_dpm_sclk marked '*'
double read_sclk_mhz(const std::string& path)
{
    std::ifstream f(path);
    std::string line;
    while (std::getline(f, line))
        if (!line.empty() && line.back() == '*') return std::atof(line.c_str() + line.find(':') + 1);
    return -1.0;
}

double read_number(const std::string& path)
{
    std::ifstream f(path);
    double v = -1.0;
    f >> v;
    return f ? v : -1.0;
}

struct Sample {
    double mhz, watts;
};

template <int KIND, bool LDS_FEED>
void run_case(const u32x4* src, float* out, const char* name, double seconds)
{
    constexpr int NF = KIND == 0 ? 4 : 8;
    constexpr double kFlopPerSweepWave = NF * NF * (KIND == 0 ? 32.0 * 32 * 16 : 16.0 * 16 * 32) * 2;
    auto launch = [&](int iters) {
        hipLaunchKernelGGL((mfma_loop<KIND, LDS_FEED>), dim3(kBlocks), dim3(kWaves * 64), 0, 0, src, iters, out);
        CHECK(hipGetLastError());
    };
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    // size one launch to about 20 ms
    int iters = 2000;
    launch(iters);
    CHECK(hipDeviceSynchronize());
    float ms = 0.f;
    CHECK(hipEventRecord(e0));
    launch(iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    iters = std::max(2, (int)(iters * 20.0 / std::max(ms, 1e-3f))) & ~1;

    const std::string sclk = first_match("/sys/class/drm/card*/device/pp_dpm_sclk");
    std::string power = first_match("/sys/class/drm/card*/device/hwmon/hwmon*/power1_average");
    if (power.empty()) power = first_match("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input");
    std::atomic<bool> stop{false}, timing{false};
    std::vector<Sample> samples;
    std::thread sampler([&] {
        while (!stop.load()) {
            if (timing.load())
                samples.push_back({sclk.empty() ? -1.0 : read_sclk_mhz(sclk),
                                   power.empty() ? -1.0 : read_number(power) / 1e6});
            std::this_thread::sleep_for(std::chrono::milliseconds(20));
        }
    });
    // settle the clock under this load, then time `seconds` of launches
    const auto t0 = std::chrono::steady_clock::now();
    while (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() < 1.5) {
        launch(iters);
        CHECK(hipDeviceSynchronize());
    }
    const int reps = std::max(1, (int)(seconds * 1e3 / 20.0));
    timing = true;
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) launch(iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    timing = false;
    stop = true;
    sampler.join();
    CHECK(hipEventElapsedTime(&ms, e0, e1));

    double mhz = 0, watts = 0;
    int nm = 0, nw = 0;
    for (const Sample& s : samples) {
        if (s.mhz > 0) mhz += s.mhz, ++nm;
        if (s.watts > 0) watts += s.watts, ++nw;
    }
    mhz = nm ? mhz / nm : -1;
    watts = nw ? watts / nw : -1;
    const double tflops = kFlopPerSweepWave * iters * kBlocks * kWaves * reps / (ms * 1e-3) / 1e12;
    const double per_ghz = mhz > 0 ? tflops / (mhz / 1e3) : -1;
    std::printf("%-44s %7.1f TFLOP/s (%.3f of 2516.6)  sclk %5.0f MHz  %6.1f TFLOP/s per GHz (%4.1f %%)  "
                "%5.0f W  %.3f pJ/FLOP\n",
                name, tflops, tflops / 2516.6, mhz, per_ghz, per_ghz > 0 ? 100 * per_ghz / kPerGhz : -1, watts,
                watts > 0 ? watts / tflops : -1);
    std::fflush(stdout);
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014)
uint64_t splitmix64(uint64_t& state)
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

}  // namespace

int main(int argc, char** argv)
{
    const double seconds = argc > 1 ? std::atof(argv[1]) : 1.0;
    if (!(seconds > 0 && seconds <= 30)) {
        std::fprintf(stderr, "usage: %s [seconds per case, (0, 30]]\n", argv[0]);
        return 2;
    }
    const size_t nvec = (size_t)kBlocks * kWaves * kFrags * 64;  // 16-byte vectors
    std::vector<uint16_t> rnd(nvec * 8), one(nvec * 8, 0x3C00);  // 0x3C00 = 1.0
    uint64_t state = 20260101;
    for (uint16_t& h : rnd) {
        const uint64_t x = splitmix64(state);
        const uint16_t sign = (uint16_t)((x >> 63) << 15);
        const uint16_t expo = (uint16_t)(13 + ((x >> 32) & 3));  // 2^-2 .. 2^1
        h = (uint16_t)(sign | (expo << 10) | (x & 0x3FF));
    }
    u32x4 *d_rnd, *d_one;
    float* d_out;
    CHECK(hipMalloc(&d_rnd, nvec * 16));
    CHECK(hipMalloc(&d_one, nvec * 16));
    CHECK(hipMalloc(&d_out, (size_t)kBlocks * kWaves * 64 * sizeof(float)));
    CHECK(hipMemcpy(d_rnd, rnd.data(), nvec * 16, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(d_one, one.data(), nvec * 16, hipMemcpyHostToDevice));

    run_case<0, false>(d_rnd, d_out, "32x32x16, random operands, registers", seconds);
    run_case<0, true>(d_rnd, d_out, "32x32x16, random operands, from LDS", seconds);
    run_case<1, false>(d_rnd, d_out, "16x16x32, random operands, registers", seconds);
    run_case<0, false>(d_one, d_out, "32x32x16, constant operands, registers", seconds);
    run_case<0, true>(d_one, d_out, "32x32x16, constant operands, from LDS", seconds);
    run_case<0, false>(d_rnd, d_out, "32x32x16, random operands, registers (again)", seconds);

    CHECK(hipFree(d_rnd));
    CHECK(hipFree(d_one));
    CHECK(hipFree(d_out));
    return 0;
}
